"""GPU check of the previous-layer reuse schedule (Multi-layer Indexer post):
layer l >= 1 attends over layer l-1's top-k, layer 0 over its own; the
overlapped schedule (indexer on a second stream) gives bit-identical outputs
to the same schedule on one stream, and each layer matches the CPU oracle's
attention over the oracle's selection (attention tolerance as in the sparse
attention tests: 2^-7 * max|v| + 1e-5 per element)."""
import numpy as np
import pytest

import csa_inputs
import oracle

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import lightning_indexer_top_02_amd as L  # noqa: E402


def _say(msg):
    print(f"[csa-test] {msg}", flush=True)


def _bf(x):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()


def _layers(n, B, S_q, T, topk, seed):
    out = []
    for li in range(n):
        pi = csa_inputs.make_integer(B=B, S_q=S_q, T=T, H=64, D=128, m=4, topk=topk, q_pos0=4 * T - S_q,
                                     seed=seed + li, qk_range=2, w_range=2)
        pi["q"] = csa_inputs.f32_to_bf16_bits(pi["q"])
        pi["k"] = csa_inputs.f32_to_bf16_bits(pi["k"])
        pi["dtype"] = "bf16"
        pa = csa_inputs.make_attention(B, S_q, T, n_sel=8, seed=seed + 100 + li)
        out.append((pi, pa))
    return out


@pytest.mark.parametrize("S_q", [1, 24])          # decode entry, and prefill entry above 16 rows
def test_mli_schedule_matches_oracle(S_q):
    B, T, topk = 2, 600, 96
    probs = _layers(4, B, S_q, T, topk, seed=41)
    dev = [((_bf(pi["q"]), _bf(pi["k"]), torch.from_numpy(pi["w"]).cuda()),
            (_bf(pa["q"]), _bf(pa["k"]), _bf(pa["v"]))) for pi, pa in probs]
    q_pos0 = probs[0][0]["q_pos0"]
    _say(f"MLI schedule: 4 layers, B={B} S_q={S_q} T={T} topk={topk}")
    outs = {}
    for ov in (True, False):
        res = L.MultiLayerIndexer(topk=topk, overlap=ov).run(dev, m=4, q_pos0=q_pos0)
        torch.cuda.synchronize()
        outs[ov] = [o.cpu().numpy() for o in res]
    for a, b in zip(outs[True], outs[False]):
        assert np.array_equal(a, b)
    sels = [oracle.oracle_topk(pi, topk)[0] for pi, _ in probs]
    for li, (pi, pa) in enumerate(probs):
        sel = sels[max(li - 1, 0)]
        ref = oracle.oracle_attention(pa, sel, pa["scale"])
        vv = oracle.decode_bf16(pa["v"])
        for b in range(B):
            for t in range(S_q):
                s = sel[b, t][sel[b, t] >= 0]
                tol = 2.0 ** -7 * np.abs(vv[b, s]).max(axis=0)[None, :] + 1e-5
                assert (np.abs(outs[True][li][b, t] - ref[b, t]) <= tol).all(), f"layer {li} row ({b},{t})"
