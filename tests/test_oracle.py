"""Pins for the CPU oracle (no GPU).

The source pages print no worked example, so the oracle is pinned to
mathematics it must reproduce: hand-derived closed forms, special cases that
reduce to a library routine, exhaustive enumeration on tiny inputs, and
invariants.  ``test_pins_catch_planted_mistakes`` plants plausible mistakes
in the oracle (on the CPU) and checks that some pin fails for each.
"""
import math

import numpy as np
import pytest

import csa_inputs
import oracle
from oracle import csa_oracle


def _prob(q, k, w, m=4, q_pos0=0, topk=4, dtype="f32", kv_len=None, causal=True):
    q = np.asarray(q, dtype=np.float32)
    k = np.asarray(k, dtype=np.float32)
    w = np.asarray(w, dtype=np.float32)
    B, S_q, H, D = q.shape
    return dict(dtype=dtype, B=B, S_q=S_q, T=k.shape[1], H=H, D=D, m=m, q_pos0=q_pos0,
                topk=topk, q=q, k=k, w=w, kv_len=kv_len, causal=causal)


def _linear_scores_problem(T, S_q, m, q_pos0, topk, slope=1.0):
    """H=1, D=1, w=1, q=1, k[s]=slope*s  =>  I[s] = max(slope*s, 0)."""
    q = np.ones((1, S_q, 1, 1))
    k = (slope * np.arange(T, dtype=np.float64)).reshape(1, T, 1)
    w = np.ones((1, S_q, 1))
    return _prob(q, k, w, m=m, q_pos0=q_pos0, topk=topk)


def _signed_problem(vals, S_q=1, q_pos0=10**6, topk=4):
    """Two heads with q=+1,w=+1 and q=-1,w=-1, D=1, k[s]=vals[s]
    => I[s] = relu(v) - relu(-v) = v exactly."""
    T = len(vals)
    q = np.zeros((1, S_q, 2, 1))
    q[:, :, 0, 0] = 1.0
    q[:, :, 1, 0] = -1.0
    w = np.zeros((1, S_q, 2))
    w[:, :, 0] = 1.0
    w[:, :, 1] = -1.0
    k = np.asarray(vals, dtype=np.float64).reshape(1, T, 1)
    return _prob(q, k, w, m=4, q_pos0=q_pos0, topk=topk)


# ---------------------------------------------------------------------------
# pins (each raises AssertionError on failure; reused by the mutation test)


def pin_bf16_decode():
    bits = np.array([0x3F80, 0xC040, 0x0000, 0x8000, 0x3F81, 0x7F7F, 0x0001], dtype=np.uint16)
    got = oracle.decode_bf16(bits)
    want = [1.0, -3.0, 0.0, -0.0, 1.0 + 2.0 ** -7, (2.0 - 2.0 ** -7) * 2.0 ** 127, 2.0 ** -133]
    assert list(got) == want
    assert np.signbit(got[3]) and not np.signbit(got[2])


def pin_rank1_closed_form():
    # q[j] = a_j * e0, k[s] = b_s * e0  =>  L[j,s] = a_j b_s,
    # I[s] = sum_j w_j max(a_j b_s, 0).  a=(1,-2,3), w=(0.5,1,-1):
    #   b= 2: relu(2,-4,6)   -> 0.5*2 + 0 - 6  = -5
    #   b=-1: relu(-1,2,-3)  -> 0 + 2 + 0      =  2
    #   b= 0:                                     0
    #   b= 1: relu(1,-2,3)   -> 0.5 + 0 - 3    = -2.5
    #   b=-3: relu(-3,6,-9)  -> 6
    a = [1.0, -2.0, 3.0]
    b = [2.0, -1.0, 0.0, 1.0, -3.0]
    q = np.zeros((1, 1, 3, 4))
    q[0, 0, :, 0] = a
    k = np.zeros((1, 5, 4))
    k[0, :, 0] = b
    w = np.array([0.5, 1.0, -1.0]).reshape(1, 1, 3)
    p = _prob(q, k, w, q_pos0=100, topk=3)
    idx, sc, vis = oracle.oracle_topk(p)
    assert vis[0, 0] == 5
    assert idx[0, 0].tolist() == [4, 1, 2]
    assert sc[0, 0].tolist() == [6.0, 2.0, 0.0]
    p5 = dict(p, topk=5)
    idx5, sc5, _ = oracle.oracle_topk(p5)
    assert idx5[0, 0].tolist() == [4, 1, 2, 3, 0]
    assert sc5[0, 0].tolist() == [6.0, 2.0, 0.0, -2.5, -5.0]


def pin_basis_closed_form():
    # q[0]=e0, q[1]=e1 (D=3), w=(1,-2): I[s] = relu(k[s,0]) - 2 relu(k[s,1])
    #   k0=( 1, 2,7): 1-4 = -3 ; k1=(-1,3,0): 0-6 = -6
    #   k2=( 2,-5,1): 2-0 =  2 ; k3=( 0,0,9): 0
    q = np.zeros((1, 1, 2, 3))
    q[0, 0, 0, 0] = 1.0
    q[0, 0, 1, 1] = 1.0
    k = np.array([[1, 2, 7], [-1, 3, 0], [2, -5, 1], [0, 0, 9]], dtype=np.float64).reshape(1, 4, 3)
    w = np.array([1.0, -2.0]).reshape(1, 1, 2)
    p = _prob(q, k, w, q_pos0=100, topk=4)
    idx, sc, _ = oracle.oracle_topk(p)
    assert idx[0, 0].tolist() == [2, 3, 0, 1]
    assert sc[0, 0].tolist() == [2.0, 0.0, -3.0, -6.0]


def pin_causal_boundary():
    # I[s] = s, so row t keeps the n = min(k, vis) highest visible indices,
    # vis = min(floor(t/m) + 1, T).
    for m, q_pos0 in [(4, 0), (4, 5), (3, 17), (1, 0)]:
        p = _linear_scores_problem(T=64, S_q=300, m=m, q_pos0=q_pos0, topk=6)
        idx, _, vis = oracle.oracle_topk(p)
        for i in range(300):
            v = min((q_pos0 + i) // m + 1, 64)
            assert vis[0, i] == v
            n = min(6, v)
            want = list(range(v - 1, v - 1 - n, -1)) + [-1] * (6 - n)
            assert idx[0, i].tolist() == want, (m, q_pos0, i)


def pin_signed_zero_and_negative_weight():
    # w = -1, q = 1, k[s] = s  =>  I[s] = -max(s,0) = -s, and I[0] = -0 -> +0.
    p = _linear_scores_problem(T=10, S_q=1, m=1, q_pos0=50, topk=4)
    p["w"] = -p["w"]
    idx, sc, _ = oracle.oracle_topk(p)
    assert idx[0, 0].tolist() == [0, 1, 2, 3]
    assert sc[0, 0].tolist() == [0.0, -1.0, -2.0, -3.0]
    assert not np.signbit(sc[0, 0, 0])


def pin_tie_floods():
    # all-zero q: I == 0 everywhere -> the n lowest indices
    rng = np.random.default_rng(7)
    q = np.zeros((1, 3, 4, 8))
    k = rng.integers(-3, 4, size=(1, 40, 8))
    w = rng.integers(-2, 3, size=(1, 3, 4))
    p = _prob(q, k, w, m=1, q_pos0=35, topk=5)
    idx, _, _ = oracle.oracle_topk(p)
    for i in range(3):
        assert idx[0, i].tolist() == [0, 1, 2, 3, 4]
    # constant keys: every visible key has the same score
    q = rng.integers(-3, 4, size=(1, 3, 4, 8))
    k = np.tile(rng.integers(-3, 4, size=(1, 1, 8)), (1, 40, 1))
    p = _prob(q, k, w, m=1, q_pos0=35, topk=5)
    idx, _, _ = oracle.oracle_topk(p)
    for i in range(3):
        assert idx[0, i].tolist() == [0, 1, 2, 3, 4]


def pin_single_head_stable_argsort():
    # H=1, w=1, non-negative inputs: I = K q, ranking = stable descending argsort.
    rng = np.random.default_rng(11)
    for trial in range(5):
        T, D = 50, 5
        q = rng.integers(0, 4, size=(1, 1, 1, D)).astype(np.float64)
        k = rng.integers(0, 4, size=(1, T, D)).astype(np.float64)
        p = _prob(q, k, np.ones((1, 1, 1)), m=1, q_pos0=10**4, topk=12)
        idx, _, _ = oracle.oracle_topk(p)
        x = k[0] @ q[0, 0, 0]
        want = np.argsort(-x, kind="stable")[:12]
        assert idx[0, 0].tolist() == want.tolist()


def pin_exhaustive():
    for seed in range(12):
        rng = np.random.default_rng(100 + seed)
        S_q, T, H, D = 5, 8, 2, 3
        q = rng.integers(-2, 3, size=(1, S_q, H, D))
        k = rng.integers(-2, 3, size=(1, T, D))
        w = rng.integers(-1, 2, size=(1, S_q, H))
        p = _prob(q, k, w, m=1, q_pos0=3, topk=4)
        idx, sc, vis = oracle.oracle_topk(p)
        for i in range(S_q):
            v = int(vis[0, i])
            ex = oracle.exact_int_scores(q[0, i], k[0, :v], w[0, i])
            best = oracle.exhaustive_topk(ex, 4)
            got = sorted(x for x in idx[0, i].tolist() if x >= 0)
            assert tuple(got) == best, (seed, i)
            n = len(best)
            assert [float(ex[j]) for j in idx[0, i, :n]] == sc[0, i, :n].tolist()


def pin_threshold_closed_form():
    vals = [float(s - 10) for s in range(20)]           # I[s] = s - 10 exactly
    p = _signed_problem(vals, topk=20)
    idx, cnt, _ = oracle.oracle_threshold(p, 0.5, 0.0, cap=20)
    assert cnt[0, 0] == 9 and idx[0, 0, :9].tolist() == list(range(19, 10, -1))
    idx, cnt, _ = oracle.oracle_threshold(p, 0.5, 2.5, cap=20)   # theta = -2.5
    assert cnt[0, 0] == 12
    tau = 1.0 / (1.0 + math.exp(-3.5))                   # theta = 3.5
    assert abs(oracle.logit_threshold(tau, 0.0) - 3.5) < 1e-5
    idx, cnt, _ = oracle.oracle_threshold(p, tau, 0.0, cap=20)
    assert cnt[0, 0] == 6 and idx[0, 0, :6].tolist() == [19, 18, 17, 16, 15, 14]
    idx, cnt, _ = oracle.oracle_threshold(p, 0.5, 0.0, cap=4)
    assert cnt[0, 0] == 9 and idx[0, 0].tolist() == [19, 18, 17, 16]


def pin_interleaved_closed_form():
    # I[s] = s, T = 16, P = 4: partition p = {p, p+4, p+8, p+12}
    p = _linear_scores_problem(T=16, S_q=1, m=1, q_pos0=100, topk=8)
    il, _ = oracle.oracle_interleaved(p, 4, 2)
    assert il[0, 0].tolist() == [12, 8, 13, 9, 14, 10, 15, 11]
    g, _, _ = oracle.oracle_topk(p)
    assert oracle.oracle_recall(il[0], g[0]).tolist() == [1.0]
    il1, _ = oracle.oracle_interleaved(p, 4, 1)
    assert il1[0, 0].tolist() == [12, 13, 14, 15]
    assert oracle.oracle_recall(il1[0], g[0]).tolist() == [0.5]
    # skewed: I[s] = s + 100*[s mod 4 == 0]; G = {12,8,4,0,15,14,13,11}
    q = np.ones((1, 1, 1, 2))
    k = np.stack([np.arange(16.0), 100.0 * (np.arange(16) % 4 == 0)], axis=1).reshape(1, 16, 2)
    p2 = _prob(q, k, np.ones((1, 1, 1)), m=1, q_pos0=100, topk=8)
    g2, _, _ = oracle.oracle_topk(p2)
    assert sorted(g2[0, 0].tolist()) == [0, 4, 8, 11, 12, 13, 14, 15]
    il2, _ = oracle.oracle_interleaved(p2, 4, 2)
    assert il2[0, 0].tolist() == [12, 8, 13, 9, 14, 10, 15, 11]
    assert oracle.oracle_recall(il2[0], g2[0]).tolist() == [0.75]


ALL_PINS = [pin_bf16_decode, pin_rank1_closed_form, pin_basis_closed_form, pin_causal_boundary,
            pin_signed_zero_and_negative_weight, pin_tie_floods, pin_single_head_stable_argsort,
            pin_exhaustive, pin_threshold_closed_form, pin_interleaved_closed_form]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


# ---------------------------------------------------------------------------
# planted mistakes: each must make at least one pin fail


def _mut_no_relu(q, k, w):
    return (w[:, None] * (q @ k.T)).sum(0) + 0.0


def _mut_relu_after_sum(q, k, w):
    return np.maximum((w[:, None] * (q @ k.T)).sum(0), 0.0) + 0.0


def _mut_relu_of_weighted(q, k, w):
    return np.maximum(w[:, None] * (q @ k.T), 0.0).sum(0) + 0.0


def _mut_sign(q, k, w):
    return -(w[:, None] * np.maximum(q @ k.T, 0.0)).sum(0) + 0.0


def _mut_abs_weights(q, k, w):
    return (np.abs(w)[:, None] * np.maximum(q @ k.T, 0.0)).sum(0) + 0.0


def _vis_off_by_one(t_abs, m, T, causal=True, kv_len=None):
    vis = (t_abs // m) if causal else T
    vis = min(vis, T)
    if kv_len is not None:
        vis = min(vis, max(int(kv_len), 0))
    return max(vis, 0)


def _select_high_ties(I, n):
    vis = I.shape[0]
    n = min(n, vis)
    if n <= 0:
        return np.zeros(0, dtype=np.int64)
    v = np.partition(I, vis - n)[vis - n]
    above = np.nonzero(I > v)[0]
    equal = np.nonzero(I == v)[0][::-1]
    sel = np.concatenate([above, equal[: n - above.shape[0]]])
    return csa_oracle.order_desc(I, sel)


def _interleave_by_block(prob, P, k_local, rows=None):
    # wrong partitioning: contiguous blocks instead of s mod P
    rows = np.arange(prob["S_q"]) if rows is None else rows
    out = np.full((prob["B"], len(rows), P * k_local), -1, dtype=np.int32)
    wd = csa_oracle._Widened(prob)
    for b in range(prob["B"]):
        for r, i in enumerate(rows):
            I = wd.scores(b, int(i))
            vis = I.shape[0]
            size = -(-vis // P)
            for p in range(P):
                part = np.arange(p * size, min(vis, (p + 1) * size))
                if part.shape[0] == 0:
                    continue
                sel = part[csa_oracle.select_topk(I[part], k_local)]
                out[b, r, p * k_local: p * k_local + sel.shape[0]] = sel
    return out, None


MUTANTS = {
    "no_relu": ("row_scores", _mut_no_relu),
    "relu_after_sum": ("row_scores", _mut_relu_after_sum),
    "relu_of_weighted": ("row_scores", _mut_relu_of_weighted),
    "sign": ("row_scores", _mut_sign),
    "abs_weights": ("row_scores", _mut_abs_weights),
    "vis_off_by_one": ("visible_count", _vis_off_by_one),
    "ties_high": ("select_topk", _select_high_ties),
}


def _pins_fail():
    failed = []
    for pin in ALL_PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    return failed


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistakes(monkeypatch, name):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(csa_oracle, attr, fn)
    assert _pins_fail(), f"no pin caught mutant {name}"


def test_pins_catch_wrong_interleave(monkeypatch):
    monkeypatch.setattr(oracle, "oracle_interleaved", _interleave_by_block)
    with pytest.raises(AssertionError):
        pin_interleaved_closed_form()


# ---------------------------------------------------------------------------
# invariants and special cases on the named workloads


def _check_topk_invariants(I_rows, idx, vis, topk):
    for r in range(idx.shape[0]):
        v = int(vis[r])
        n = min(topk, v)
        sel = idx[r, :n]
        assert (idx[r, n:] == -1).all()
        assert (sel >= 0).all() and (sel < v).all()
        assert len(set(sel.tolist())) == n
        if n < v:
            I = I_rows[r]
            mask = np.ones(v, dtype=bool)
            mask[sel] = False
            lo, hi = I[sel].min(), I[mask].max()
            assert lo >= hi
            if lo == hi:       # ties at the cut go to the lower index
                assert sel[I[sel] == lo].max() < np.nonzero(mask & (I == hi))[0].min()


def test_config1_invariants_and_exact_scores():
    p = csa_inputs.config(1)
    idx, sc, vis = oracle.oracle_topk(p)
    wd = csa_oracle._Widened(p)
    I_rows = [wd.scores(0, i) for i in range(p["S_q"])]
    _check_topk_invariants(I_rows, idx[0], vis[0], p["topk"])
    # scores are exact integers; cross-check a few rows with Python integers
    for i in [0, 255, 256, 600, 1023]:
        v = int(vis[0, i])
        ex = oracle.exact_int_scores(p["q"][0, i], p["k"][0, :v], p["w"][0, i])
        n = min(p["topk"], v)
        assert [float(ex[j]) for j in idx[0, i, :n]] == sc[0, i, :n].tolist()


def test_rows_with_few_visible_keys_closed_form():
    p = csa_inputs.config(1)
    idx, _, vis = oracle.oracle_topk(p, rows=np.arange(0, 300))
    for r in range(300):
        v = int(vis[0, r])
        if v <= p["topk"]:
            assert sorted(idx[0, r, :v].tolist()) == list(range(v))
            assert (idx[0, r, v:] == -1).all()


def test_head_permutation_and_weight_scale():
    p = csa_inputs.make_integer(S_q=64, T=40, H=6, D=8, m=1, topk=10, seed=5)
    idx0, sc0, _ = oracle.oracle_topk(p)
    perm = np.random.default_rng(3).permutation(6)
    pp = dict(p, q=p["q"][:, :, perm, :].copy(), w=p["w"][:, :, perm].copy())
    idx1, sc1, _ = oracle.oracle_topk(pp)
    assert (idx0 == idx1).all() and (sc0 == sc1).all()
    ps = dict(p, w=p["w"] * 3)
    idx2, sc2, _ = oracle.oracle_topk(ps)
    assert (idx0 == idx2).all()
    fin = np.isfinite(sc0)
    assert (sc2[fin] == 3 * sc0[fin]).all()
    # scaling w changes the threshold variant when theta != 0
    vals = [float(s - 10) for s in range(20)]
    q = _signed_problem(vals, topk=20)
    q3 = dict(q, w=q["w"] * 3)
    _, c1, _ = oracle.oracle_threshold(q, 0.5, 2.5, cap=20)
    _, c3, _ = oracle.oracle_threshold(q3, 0.5, 2.5, cap=20)
    assert c1[0, 0] == 12 and c3[0, 0] == 10


def test_kv_len_and_noncausal():
    p = _linear_scores_problem(T=30, S_q=40, m=1, q_pos0=0, topk=5)
    p["kv_len"] = np.array([7])
    idx, _, vis = oracle.oracle_topk(p)
    for i in range(40):
        v = min(i + 1, 7)
        assert vis[0, i] == v
        n = min(5, v)
        assert idx[0, i, :n].tolist() == list(range(v - 1, v - 1 - n, -1))
    p["kv_len"] = None
    p["causal"] = False
    idx, _, vis = oracle.oracle_topk(p)
    assert (vis == 30).all() and (idx[0, :, 0] == 29).all()


def test_threshold_nesting_and_cap():
    p = csa_inputs.make_gaussian_bf16(1, 16, 200, 8, 32, 1, 50, q_pos0=300, seed=9)
    prev = None
    for tau in [0.3, 0.5, 0.51, 0.6]:
        idx, cnt, _ = oracle.oracle_threshold(p, tau, 0.0, cap=200)
        sets = [set(x for x in idx[0, r].tolist() if x >= 0) for r in range(16)]
        if prev is not None:
            assert all(s <= t for s, t in zip(sets, prev))
        prev = sets
    full, cnt, _ = oracle.oracle_threshold(p, 0.5, 0.0, cap=200)
    capd, cnt2, _ = oracle.oracle_threshold(p, 0.5, 0.0, cap=7)
    assert (cnt == cnt2).all()
    assert (capd[0] == full[0, :, :7]).all()


def test_interleaved_recall_closed_form_random():
    p = csa_inputs.make_gaussian_bf16(1, 8, 512, 8, 32, 1, 64, q_pos0=600, seed=13)
    g, _, _ = oracle.oracle_topk(p)
    for P, kl in [(1, 64), (4, 10), (8, 4), (8, 64)]:
        il, _ = oracle.oracle_interleaved(p, P, kl)
        rec = oracle.oracle_recall(il[0], g[0])
        for r in range(8):
            G = set(g[0, r].tolist())
            cp = [sum(1 for s in G if s % P == part) for part in range(P)]
            assert rec[r] == sum(min(c, kl) for c in cp) / len(G)
        if P == 1:
            assert (np.sort(il[0], axis=1) == np.sort(g[0], axis=1)).all()
        if kl >= 64:
            assert (rec == 1.0).all()


def test_decode_planted_keys_selected():
    p = csa_inputs.make_decode(B=2, context=4096, topk=128, n_planted=16, seed=77)
    idx, _, vis = oracle.oracle_topk(p)
    assert (vis == 1024).all()
    for b in range(2):
        assert set(p["planted"][b].tolist()) <= set(idx[b, 0].tolist())
