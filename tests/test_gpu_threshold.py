"""GPU parity of csa_index_threshold_select (sigmoid threshold instead of top-k)."""
import math

import numpy as np
import pytest

import csa_inputs
import oracle

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import lightning_indexer_top_02_amd as L  # noqa: E402
from gpu_common import REL, FLOOR_DIV, check_exact, to_device  # noqa: E402


def _thr(prob, cap, tau, bias, **kw):
    q, k, w, kv = to_device(prob)
    idx, cnt, sc = L.index_threshold_select(q, k, w, cap, prob_threshold=tau, logit_bias=bias, m=prob["m"],
                                            q_pos0=prob["q_pos0"], kv_len=kv, return_scores=True,
                                            causal=prob.get("causal", True), **kw)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), cnt.cpu().numpy(), sc.cpu().numpy()


def _integer(S_q=200, T=600, seed=4, H=64, D=128, bf16=True):
    p = csa_inputs.make_integer(S_q=S_q, T=T, H=H, D=D, m=4, topk=64, q_pos0=1500, seed=seed,
                                qk_range=2, w_range=2)
    if bf16:
        p["q"] = csa_inputs.f32_to_bf16_bits(p["q"])
        p["k"] = csa_inputs.f32_to_bf16_bits(p["k"])
        p["dtype"] = "bf16"
    return p


@pytest.mark.parametrize("tau,bias,cap", [(0.5, 0.0, 600), (0.5, 0.0, 37), (0.5, 2.5, 128),
                                          (1 / (1 + math.exp(-3.5)), 0.0, 256), (0.2, -1.0, 64)])
@pytest.mark.parametrize("bf16", [True, False])
def test_threshold_exact_integer(tau, bias, cap, bf16):
    p = _integer(bf16=bf16) if bf16 else _integer(H=4, D=32, bf16=False)
    ref_i, ref_c, ref_s = oracle.oracle_threshold(p, tau, bias, cap)
    idx, cnt, sc = _thr(p, cap, tau, bias)
    assert (cnt == ref_c).all()
    check_exact(idx, ref_i, sc, ref_s)


def test_threshold_half_is_sign_test():
    # tau = 0.5, bias = 0 keeps exactly the keys with I > 0 (strict)
    p = _integer()
    idx, cnt, _ = _thr(p, 600, 0.5, 0.0)
    scorer = oracle.RowScorer(p)
    for r in range(p["S_q"]):
        I = scorer(0, r)
        assert cnt[0, r] == int((I > 0).sum())


@pytest.mark.parametrize("cap", [512, 40])
def test_threshold_bf16_gaussian_tolerance(cap):
    """Gaussian bf16 inputs: the count, the returned scores and the kept set
    under the bf16 tolerance rule.  With cap = 512 most rows keep every
    survivor; with cap = 40 most rows truncate, and the kept keys must be the
    survivors' best 40 by score (up to the band around the 40th)."""
    p = csa_inputs.make_gaussian_bf16(1, 256, 2048, 64, 128, 4, 512, q_pos0=7000, seed=17)
    tau, bias = 0.5, -0.05
    idx, cnt, sc = _thr(p, cap, tau, bias)
    theta = oracle.logit_threshold(tau, bias)
    scorer = oracle.RowScorer(p)
    truncated = 0
    for r in range(p["S_q"]):
        I = scorer(0, r)
        floor = float(np.sqrt(np.mean(I * I))) / FLOOR_DIV
        band = REL * max(abs(theta), floor)
        near = int((np.abs(I - theta) <= band).sum())
        true_cnt = int((I > theta).sum())
        assert abs(int(cnt[0, r]) - true_cnt) <= near
        n = min(cap, int(cnt[0, r]))
        sel = idx[0, r, :n]
        assert (idx[0, r, n:] == -1).all() and len(set(sel.tolist())) == n
        assert (I[sel] > theta - band).all()
        # scores: each within the rule of its oracle score; padding -inf
        err = np.abs(sc[0, r, :n].astype(np.float64) - I[sel])
        assert (err <= REL * np.maximum(np.abs(I[sel]), floor)).all(), f"row {r}: score error {err.max()}"
        assert np.isneginf(sc[0, r, n:]).all()
        surv = oracle.order_desc(I, np.nonzero(I > theta)[0])
        if true_cnt > cap:                          # the cap keeps the survivors' best by score
            truncated += 1
            ref = surv[:cap]
            vc = I[ref].min()
            bc = REL * max(abs(vc), floor)
            for s_ in set(sel.tolist()) ^ set(ref.tolist()):
                assert abs(I[s_] - vc) <= bc, f"row {r}: index {s_} outside the band of the cap-th survivor"
        else:                                       # every survivor kept, up to keys at the threshold
            for s_ in set(sel.tolist()) ^ set(surv.tolist()):
                assert abs(I[s_] - theta) <= band, f"row {r}: survivor {s_} missing or extra"
    if cap == 40:                                   # both branches above are exercised
        assert p["S_q"] // 2 < truncated < p["S_q"]


def test_threshold_nesting_gpu():
    p = _integer()
    prev = None
    for tau in [0.3, 0.5, 0.7, 0.9]:
        idx, cnt, _ = _thr(p, 600, tau, 0.0)
        sets = [set(x for x in idx[0, r].tolist() if x >= 0) for r in range(p["S_q"])]
        if prev is not None:
            assert all(a <= b for a, b in zip(sets, prev))
        prev = sets


def _decode_integer(B=3, S_q=2, T=3000, seed=31, kv_len=None):
    """Few query rows against long key rows: the decode key scan path."""
    p = csa_inputs.make_integer(B=B, S_q=S_q, T=T, H=64, D=128, m=4, topk=64, q_pos0=4 * T - S_q, seed=seed,
                                qk_range=2, w_range=2)
    p["q"] = csa_inputs.f32_to_bf16_bits(p["q"])
    p["k"] = csa_inputs.f32_to_bf16_bits(p["k"])
    p["dtype"] = "bf16"
    if kv_len is not None:
        p["kv_len"] = np.asarray(kv_len, dtype=np.int32)
    return p


@pytest.mark.parametrize("case,cap,tau,bias", [("over_cap", 200, 0.5, 0.0),       # survivors > cap
                                               ("under_cap", 4096, 0.5, 0.0),     # every survivor fits
                                               ("high_threshold", 300, 0.5, -6.0),
                                               ("kv_len", 256, 0.5, 0.0),         # short and empty rows
                                               ("long_rows", 1024, 0.5, 2.0),     # rows past the register tile
                                               ("noncausal", 400, 0.5, 0.0)])
def test_threshold_decode_path_exact(case, cap, tau, bias):
    if case == "kv_len":
        p = _decode_integer(kv_len=[3000, 170, 0])
    elif case == "long_rows":
        p = _decode_integer(B=2, S_q=1, T=40000, seed=32)
    elif case == "noncausal":
        p = _decode_integer(S_q=4, seed=33)
        p["causal"], p["q_pos0"] = False, 0
    else:
        p = _decode_integer()
    ref_i, ref_c, ref_s = oracle.oracle_threshold(p, tau, bias, cap)
    idx, cnt, sc = _thr(p, cap, tau, bias)
    assert (cnt == ref_c).all()
    check_exact(idx, ref_i, sc, ref_s)
    idx_s, cnt_s, sc_s = _thr(p, cap, tau, bias, sorted=True)
    assert (idx_s == ref_i).all() and (cnt_s == ref_c).all()
