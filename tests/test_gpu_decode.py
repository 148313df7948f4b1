"""GPU parity of csa_index_topk_decode (HBM-bound key scan + per-row select)."""
import numpy as np
import pytest

import csa_inputs
import oracle

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import lightning_indexer_top_02_amd as L  # noqa: E402
from gpu_common import check_exact, check_tolerance, to_device  # noqa: E402


def _say(msg):
    print(f"[csa-test] {msg}", flush=True)


def _decode(prob, topk=None, **kw):
    q, k, w, kv = to_device(prob)
    topk = prob["topk"] if topk is None else topk
    out = L.index_topk_decode(q, k, w, topk, m=prob["m"], q_pos0=prob["q_pos0"], kv_len=kv,
                              causal=prob.get("causal", True), **kw)
    torch.cuda.synchronize()
    if isinstance(out, tuple):
        return out[0].cpu().numpy(), out[1].cpu().numpy()
    return out.cpu().numpy(), None


def _prefill(prob, topk=None, **kw):
    q, k, w, kv = to_device(prob)
    topk = prob["topk"] if topk is None else topk
    out = L.index_topk_prefill(q, k, w, topk, m=prob["m"], q_pos0=prob["q_pos0"], kv_len=kv,
                               causal=prob.get("causal", True), **kw)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def test_config4_decode_parity_and_planted_keys():
    p = csa_inputs.config(4)
    _say("config 4 decode B=32 T=32768 k=2048: all rows")
    idx, sc = _decode(p, return_scores=True)
    st = check_tolerance(p, np.arange(p["S_q"]), idx, sc, p["topk"])
    _say(f"  boundary swaps={st['swaps']} max rel err={st['max_rel']:.2e}")
    for b in range(p["B"]):
        assert set(p["planted"][b].tolist()) <= set(idx[b, 0].tolist()), f"sequence {b} lost a planted key"
    idx2, _ = _decode(p)
    check_tolerance(p, np.arange(p["S_q"]), idx2, None, p["topk"])


def test_decode_matches_prefill_sets():
    p = csa_inputs.make_decode(B=4, context=20000, topk=512, S_q=3, seed=41)
    a, _ = _decode(p)
    b = _prefill(p)
    for bb in range(p["B"]):
        for r in range(p["S_q"]):
            assert sorted(a[bb, r].tolist()) == sorted(b[bb, r].tolist())


def _integer_decode(B=3, S_q=2, T=3000, topk=200, seed=3):
    p = csa_inputs.make_integer(B=B, S_q=S_q, T=T, H=64, D=128, m=4, topk=topk, q_pos0=4 * T - S_q,
                                seed=seed, qk_range=2, w_range=2)
    p["q"] = csa_inputs.f32_to_bf16_bits(p["q"])
    p["k"] = csa_inputs.f32_to_bf16_bits(p["k"])
    p["dtype"] = "bf16"
    return p


@pytest.mark.parametrize("case", ["plain", "kv_len", "sorted", "few_visible", "fp32_fallback"])
def test_decode_exact_cases(case):
    p = _integer_decode()
    kw = {}
    if case == "kv_len":
        p["kv_len"] = np.array([3000, 1234, 150], dtype=np.int32)
    elif case == "sorted":
        kw["sorted"] = True
    elif case == "few_visible":
        p["q_pos0"] = 300                      # rows see ~76 keys < topk
    elif case == "fp32_fallback":
        p = csa_inputs.make_integer(B=2, S_q=4, T=700, H=4, D=32, m=4, topk=64, q_pos0=2796, seed=9)
    _say(f"decode exact case {case}")
    ref_i, ref_s, _ = oracle.oracle_topk(p)
    idx, sc = _decode(p, return_scores=True, **kw)
    check_exact(idx, ref_i, sc, ref_s)
    if case == "sorted":
        assert (idx == ref_i).all() and (sc == ref_s).all()
