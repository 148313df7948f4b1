"""GPU parity of csa_index_topk_prefill against the CPU oracle (through the C ABI)."""
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


def _run(prob, topk=None, rows=None, **kw):
    q, k, w, kv = to_device(prob)
    topk = prob["topk"] if topk is None else topk
    out = L.index_topk_prefill(q, k, w, topk, m=prob["m"], q_pos0=prob["q_pos0"], kv_len=kv,
                               causal=prob.get("causal", True), **kw)
    torch.cuda.synchronize()
    if isinstance(out, tuple):
        idx, sc = out
        return idx.cpu().numpy(), sc.cpu().numpy()
    return out.cpu().numpy(), None


def test_config1_bit_exact():
    p = csa_inputs.config(1)
    _say("config 1 (tiny exact, fp32 integers): generic kernel")
    ref_i, ref_s, _ = oracle.oracle_topk(p)
    idx, sc = _run(p, return_scores=True)
    check_exact(idx, ref_i, sc, ref_s)
    idx2, _ = _run(p)                              # index-only path
    check_exact(idx2, ref_i)


def test_config1_sorted_matches_oracle_order():
    p = csa_inputs.config(1)
    ref_i, ref_s, _ = oracle.oracle_topk(p)
    idx, sc = _run(p, return_scores=True, sorted=True)
    assert (idx == ref_i).all()
    assert (sc == ref_s).all()
    idx2, _ = _run(p, sorted=True)
    assert (idx2 == ref_i).all()


def _integer_bf16(S_q=300, T=200, topk=64, seed=21, q_pos0=0, m=4, B=1, qr=2, wr=2):
    """Integer-valued data in bf16 at the MFMA kernel's shape (H=64, D=128): exact scores."""
    p = csa_inputs.make_integer(B=B, S_q=S_q, T=T, H=64, D=128, m=m, topk=topk, q_pos0=q_pos0, seed=seed,
                                qk_range=qr, w_range=wr)
    p["q"] = csa_inputs.f32_to_bf16_bits(p["q"])
    p["k"] = csa_inputs.f32_to_bf16_bits(p["k"])
    p["dtype"] = "bf16"
    return p


def test_mfma_integer_bit_exact_and_generic_invariance():
    p = _integer_bf16(S_q=333, T=200, topk=40, q_pos0=500)
    _say("integer bf16 H=64 D=128: mfma kernel vs oracle vs generic kernel")
    ref_i, ref_s, _ = oracle.oracle_topk(p)
    idx, sc = _run(p, return_scores=True)
    check_exact(idx, ref_i, sc, ref_s)
    with L.test_options(force_generic=1):
        idx_g, sc_g = _run(p, return_scores=True)
    check_exact(idx_g, ref_i, sc_g, ref_s)


def test_compaction_invariance_integer():
    # many ties and a tiny candidate buffer: the compaction path runs constantly
    p = _integer_bf16(S_q=96, T=2000, topk=100, q_pos0=6000, qr=1, wr=1, seed=5)
    ref_i, ref_s, _ = oracle.oracle_topk(p)
    idx_a, sc_a = _run(p, return_scores=True)
    with L.test_options(cand_cap=1):
        idx_b, sc_b = _run(p, return_scores=True)
    check_exact(idx_a, ref_i, sc_a, ref_s)
    check_exact(idx_b, ref_i, sc_b, ref_s)


def test_scaled_config2_tolerance():
    # config-2 distributions at S=4096, T=1024, k=256: several 64-key tiles, a ragged tail
    p = csa_inputs.make_gaussian_bf16(1, 4096, 1024, 64, 128, 4, 256, seed=1002, name="scaled")
    _say("scaled V4-Flash prefill S=4096 T=1024 k=256")
    rows = np.arange(p["S_q"])
    idx, sc = _run(p, return_scores=True)
    st = check_tolerance(p, rows, idx, sc, p["topk"])
    _say(f"  rows={st['rows']} boundary swaps={st['swaps']} max rel score err={st['max_rel']:.2e}")
    idx2, _ = _run(p)
    check_tolerance(p, rows, idx2, None, p["topk"])


def test_determinism_and_compaction_same_sets():
    p = csa_inputs.make_gaussian_bf16(1, 1000, 3000, 64, 128, 4, 300, q_pos0=9000, seed=31)
    a, sa = _run(p, return_scores=True)
    b, sb = _run(p, return_scores=True)
    assert (a == b).all() and (sa.view(np.uint32) == sb.view(np.uint32)).all()
    with L.test_options(cand_cap=1):
        c, sc_ = _run(p, return_scores=True)
    for r in range(a.shape[1]):
        assert sorted(a[0, r].tolist()) == sorted(c[0, r].tolist())


@pytest.mark.parametrize("case", ["ragged", "kvlen_batch", "noncausal", "topk1", "topk_gt_T",
                                  "zero_q", "const_keys", "neg_w"])
def test_edge_cases_exact(case):
    if case == "ragged":
        p = _integer_bf16(S_q=37, T=150, topk=20, q_pos0=3)
    elif case == "kvlen_batch":
        p = _integer_bf16(S_q=50, T=300, topk=30, q_pos0=1000, B=3)
        p["kv_len"] = np.array([300, 17, 0], dtype=np.int32)
    elif case == "noncausal":
        p = _integer_bf16(S_q=20, T=500, topk=64)
        p["causal"] = False
    elif case == "topk1":
        p = _integer_bf16(S_q=64, T=300, topk=1, q_pos0=1200)
    elif case == "topk_gt_T":
        p = _integer_bf16(S_q=64, T=100, topk=256, q_pos0=1000)
    elif case == "zero_q":
        p = _integer_bf16(S_q=40, T=400, topk=50, q_pos0=1600)
        p["q"][:] = 0
    elif case == "const_keys":
        p = _integer_bf16(S_q=40, T=400, topk=50, q_pos0=1600)
        p["k"][:] = p["k"][:, :1, :]
    else:                       # negative weights everywhere: -0.0 from ReLU-zero heads
        p = _integer_bf16(S_q=40, T=400, topk=50, q_pos0=1600)
        p["w"] = -np.abs(p["w"]) - 1
    _say(f"edge case {case}")
    ref_i, ref_s, _ = oracle.oracle_topk(p)
    idx, sc = _run(p, return_scores=True)
    check_exact(idx, ref_i, sc, ref_s)
    idx2, _ = _run(p)
    check_exact(idx2, ref_i)
    if case in ("zero_q", "const_keys"):
        assert not np.signbit(sc[sc == 0]).any()


def test_config2_full_size_every_row():
    """V4-Flash prefill at full size (S=16384, T=4096, k=2048): every query
    row, indices and scores, under the bf16 tolerance rule."""
    p = csa_inputs.config(2)
    _say("config 2 full size (S=16384 T=4096 k=2048): all 16384 rows")
    idx, sc = _run(p, return_scores=True)
    st = check_tolerance(p, np.arange(p["S_q"]), idx, sc, p["topk"], say=_say)
    assert st["rows"] == p["S_q"]
    _say(f"  boundary swaps={st['swaps']} max rel err={st['max_rel']:.2e}")
    idx2, _ = _run(p)                              # index-only launch: the same sets
    for r in range(p["S_q"]):
        assert set(idx2[0, r].tolist()) == set(idx[0, r].tolist()), f"row {r}: index-only run differs"


def _tail_rows(S_q, n, seed, k, m=4, q_pos0=0):
    """n seeded rows that always include the first and last rows and, when the
    range has them, the rows around vis = k (the last rows that copy their
    visible keys and the first that need a selection)."""
    must = [0, S_q - 1]
    for i in range(S_q):
        v = (q_pos0 + i) // m + 1
        if k - 1 <= v <= k + 1:
            must.append(i)
    return csa_inputs.sample_rows(S_q, n, seed=seed, must=must)


def test_config3_long_prefill_1024_rows():
    p = csa_inputs.config(3)
    rows = _tail_rows(p["S_q"], 1024, 3, p["topk"])
    assert 8191 in rows and 8192 in rows and len(rows) == 1024
    _say("config 3 long prefill (S=65536 T=16384), 1024 seeded rows incl. first, last and vis = k")
    idx, sc = _run(p, return_scores=True)
    st = check_tolerance(p, rows, idx[:, rows], sc[:, rows], p["topk"], say=_say)
    _say(f"  boundary swaps={st['swaps']} max rel err={st['max_rel']:.2e}")


def test_config5_million_token_tail_1024_rows():
    p = csa_inputs.config(5)
    rows = _tail_rows(p["S_q"], 1024, 5, p["topk"], q_pos0=p["q_pos0"])
    assert rows[0] == 0 and rows[-1] == p["S_q"] - 1 and len(rows) == 1024
    _say("config 5 tail (S_q=8192 of 1M, T=262144), 1024 seeded rows incl. first and last")
    idx, sc = _run(p, return_scores=True)
    st = check_tolerance(p, rows, idx[:, rows], sc[:, rows], p["topk"], say=_say)
    _say(f"  boundary swaps={st['swaps']} max rel err={st['max_rel']:.2e}")


@pytest.mark.parametrize("case", ["compaction", "ragged", "kvlen_batch", "topk_gt_T", "many_items",
                                  "long_cand_list"])
def test_mfma_paths_exact(case):
    """The MFMA prefill kernel returns the oracle's sets on every path of its
    candidate lists: default capacity and the smallest one (cand_cap=1:
    compactions on almost every tile), several query blocks per workgroup,
    and lists longer than the final select's registers (k = 2200)."""
    if case == "compaction":        # 24 key tiles per row
        p = _integer_bf16(S_q=96, T=2000, topk=100, q_pos0=6000, qr=1, wr=1, seed=5)
    elif case == "ragged":
        p = _integer_bf16(S_q=37, T=150, topk=20, q_pos0=3)
    elif case == "kvlen_batch":
        p = _integer_bf16(S_q=50, T=300, topk=30, q_pos0=1000, B=3)
        p["kv_len"] = np.array([300, 17, 0], dtype=np.int32)
    elif case == "topk_gt_T":
        p = _integer_bf16(S_q=64, T=100, topk=256, q_pos0=1000)
    elif case == "many_items":      # 300 query blocks over at most 512 workgroups, light and heavy ones
        p = _integer_bf16(S_q=1200, T=700, topk=50, q_pos0=0, seed=8)
    else:                           # k=2200: candidate lists of up to 4464 keys
        p = _integer_bf16(S_q=8, T=6000, topk=2200, q_pos0=4 * 5990, seed=9)
    _say(f"mfma prefill paths: {case}")
    ref_i, ref_s, _ = oracle.oracle_topk(p)
    for opts in ({}, {"cand_cap": 1}):
        with L.test_options(**opts):
            idx, sc = _run(p, return_scores=True)
            idx2, _ = _run(p)
        check_exact(idx, ref_i, sc, ref_s)
        check_exact(idx2, ref_i)


@pytest.mark.parametrize("topk", [64, 512, 2048, 4096])
def test_topk_sweep_exact_integer(topk):
    """The pages sweep top-k among their selection parameters: k = 64 ... 4096
    (the library's largest) on integer-valued bf16 inputs at the MFMA shape,
    rows of about 6000 visible keys; prefill and decode entry points both
    return the oracle's sets and scores exactly."""
    p = _integer_bf16(S_q=48, T=6000, topk=topk, q_pos0=4 * 5980, seed=200 + topk // 64)
    _say(f"top-k sweep k={topk}: prefill S_q=48, T=6000")
    ref_i, ref_s, _ = oracle.oracle_topk(p)
    idx, sc = _run(p, return_scores=True)
    check_exact(idx, ref_i, sc, ref_s)
    d = _integer_bf16(S_q=2, T=12000, topk=topk, q_pos0=4 * 12000 - 2, seed=300 + topk // 64, B=3)
    q, k, w, _ = to_device(d)
    di, ds = L.index_topk_decode(q, k, w, topk, m=4, q_pos0=d["q_pos0"], return_scores=True)
    torch.cuda.synchronize()
    rd_i, rd_s, _ = oracle.oracle_topk(d)
    check_exact(di.cpu().numpy(), rd_i, ds.cpu().numpy(), rd_s)
