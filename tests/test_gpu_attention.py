"""GPU parity of csa_sparse_attention (softmax attention over the selected keys).

Tolerance, from the arithmetic: logits and sums are fp32 over exact bf16
products (relative error ~1e-6); the softmax weights are rounded to bf16
(8 significant bits: relative error <= 2^-8 each) and the normaliser sums the
rounded weights, so the output is an exact convex combination whose weights
are off by at most 2 * 2^-8 relative, i.e. their absolute errors sum to at
most 2^-7.  Hence, per output element,
    |o_gpu - o_ref| <= 2^-7 * max_e |v[idx_e, d]| + 1e-5,
with max_e over the row's valid entries.  Cases whose weights are exactly
representable (one dominant key, equal logits) are checked to 1e-5.
"""
import numpy as np
import pytest

import csa_inputs
import oracle

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import lightning_indexer_top_02_amd as L  # noqa: E402


def _say(msg):
    print(f"[csa-test] {msg}", flush=True)


def _dev(p):
    def bf(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return bf(p["q"]), bf(p["k"]), bf(p["v"]), torch.from_numpy(np.ascontiguousarray(p["idx"])).cuda()


def _run(p, scale=None):
    q, k, v, idx = _dev(p)
    o = L.sparse_attention(q, k, v, idx, scale=p["scale"] if scale is None else scale)
    torch.cuda.synchronize()
    return o.cpu().numpy()


def _check(p, o, rows=None):
    ref = oracle.oracle_attention(p, p["idx"], p["scale"], rows=rows)
    vv = oracle.decode_bf16(p["v"])
    T = p["T"]
    worst = 0.0
    for b in range(p["B"]):
        for t in (range(p["S_q"]) if rows is None else rows):
            sel = p["idx"][b, t]
            sel = sel[(sel >= 0) & (sel < T)]
            vmax = np.abs(vv[b, sel]).max(axis=0) if len(sel) else np.zeros(p["Dv"])
            tol = 2.0 ** -7 * vmax[None, :] + 1e-5
            err = np.abs(o[b, t] - ref[b, t])
            assert (err <= tol).all(), f"row ({b},{t}): max err {err.max():.3e} over tolerance"
            worst = max(worst, float((err / tol).max()))
    return worst


@pytest.mark.parametrize("case", ["ragged_chunks", "short_rows", "many_rows", "invalid_entries",
                                  "chunks_per_workgroup"])
def test_attention_matches_oracle(case):
    if case == "ragged_chunks":        # chunks of 256 and 44 entries; -1 padding at the end
        p = csa_inputs.make_attention(2, 3, 1000, n_sel=300, seed=11, pad=10)
    elif case == "short_rows":         # fewer entries than one chunk
        p = csa_inputs.make_attention(3, 2, 500, n_sel=37, seed=12)
    elif case == "many_rows":          # more rows than workgroups: one workgroup per row
        p = csa_inputs.make_attention(2, 160, 700, n_sel=200, seed=13, pad=3)
    elif case == "chunks_per_workgroup":  # 600 rows -> one workgroup per row walks all 3 chunks
        p = csa_inputs.make_attention(2, 300, 2000, n_sel=700, seed=18, pad=7)
        p["idx"][1, 5, :300] = -1                                        # first chunk of a row empty
    else:                              # entries >= T and < -1 are skipped like -1
        p = csa_inputs.make_attention(2, 2, 400, n_sel=260, seed=14)
        p["idx"][0, 0, ::7] = 400 + np.arange(len(p["idx"][0, 0, ::7]), dtype=np.int32)
        p["idx"][1, 1, ::5] = -17
    _say(f"attention case {case}: B={p['B']} S_q={p['S_q']} T={p['T']} n_sel={p['n_sel']}")
    o = _run(p)
    _say(f"  worst err / tolerance = {_check(p, o):.3f}")


def test_attention_empty_rows_are_zero():
    p = csa_inputs.make_attention(1, 3, 300, n_sel=140, seed=15)
    p["idx"][0, 1, :] = -1
    p["idx"][0, 2, :] = 300
    o = _run(p)
    assert (o[0, 1] == 0).all() and (o[0, 2] == 0).all()
    _check(p, o)


def test_attention_exact_weights():
    """One dominant key returns its value row; a zero query averages the rows."""
    p = csa_inputs.make_attention(1, 2, 256, n_sel=150, seed=16)
    q = np.zeros((1, 2, 64, 128), np.float32)
    q[0, 0, :, 0] = 1.0                                # row 0: logit = k[s, 0] * 40
    k = oracle.decode_bf16(p["k"]).astype(np.float32)
    k[0, :, 0] = 0.0
    dom = int(p["idx"][0, 0, 77])
    k[0, dom, 0] = 8.0
    p["q"] = csa_inputs.f32_to_bf16_bits(q)            # row 1: zero query, equal logits
    p["k"] = csa_inputs.f32_to_bf16_bits(k)
    o = _run(p, scale=40.0)
    vv = oracle.decode_bf16(p["v"])
    assert np.allclose(o[0, 0], np.repeat(vv[0, dom][None], 64, 0), atol=1e-5)
    mean = vv[0, p["idx"][0, 1]].mean(0)
    assert np.allclose(o[0, 1], np.repeat(mean[None], 64, 0), atol=1e-5)


def test_attention_over_decode_selection():
    """The decode workload's own selections (B=32, T=32768, top-2048) feed the
    attention step; every row is checked against the oracle."""
    pd = csa_inputs.config(4)
    q, k, w = (torch.from_numpy(pd["q"].view(np.int16)).view(torch.bfloat16).cuda(),
               torch.from_numpy(pd["k"].view(np.int16)).view(torch.bfloat16).cuda(),
               torch.from_numpy(pd["w"]).cuda())
    sel = L.index_topk_decode(q, k, w, pd["topk"], m=pd["m"], q_pos0=pd["q_pos0"])
    torch.cuda.synchronize()
    del q, k, w
    pa = csa_inputs.make_attention(pd["B"], 1, pd["T"], n_sel=8, seed=17)
    pa["idx"] = sel.cpu().numpy()
    pa["n_sel"] = pd["topk"]
    _say("attention over the decode selection: B=32 T=32768 n_sel=2048")
    o = _run(pa)
    _say(f"  worst err / tolerance = {_check(pa, o):.3f}")
