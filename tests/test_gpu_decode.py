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


@pytest.mark.parametrize("case", ["plain", "kv_len", "sorted", "few_visible", "fp32_fallback", "max_rows",
                                  "tiny_T"])
def test_decode_exact_cases(case):
    p = _integer_decode()
    kw = {}
    if case == "max_rows":                     # the most query rows per sequence the decode path takes
        p = _integer_decode(B=2, S_q=16, T=2500, topk=300, seed=11)
    elif case == "tiny_T":                     # fewer keys than one scan step, and than k
        p = _integer_decode(B=3, S_q=3, T=5, topk=8, seed=12)
    elif case == "kv_len":
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


def _bf16_to_f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _select_case(case):
    """Decode inputs that steer the per-row select down each of its paths."""
    if case == "no_planted":          # i.i.d. scores: narrow candidate range, tiny boundary bins
        return csa_inputs.make_decode(B=3, context=131072, topk=2048, n_planted=0, seed=51)
    if case == "long_rows":           # more visible keys than the select holds in registers
        return csa_inputs.make_decode(B=2, context=4 * 40000, topk=2048, n_planted=16, seed=52)
    if case == "ragged_kv":           # partial last chunks, waves without keys, a row below topk
        p = csa_inputs.make_decode(B=4, context=4 * 9000, topk=1024, n_planted=8, S_q=2, seed=53)
        p["kv_len"] = np.array([4096 + 40, 1030, 900, 9000], dtype=np.int32)
        return p
    if case == "k_near_vis":          # topk close to the row length: waves report all their keys
        return csa_inputs.make_decode(B=2, context=4 * 3000, topk=2048, n_planted=8, seed=54)
    if case == "crowded_bin":         # all keys equal but one far above: one bin holds the rest
        p = csa_inputs.make_decode(B=2, context=4 * 20000, topk=1024, n_planted=1, seed=55)
        k = _bf16_to_f32(p["k"])
        for b in range(p["B"]):
            s = int(p["planted"][b, 0])
            top = 25.0 * k[b, s]
            k[b] = k[b, (s + 1) % p["T"]]
            k[b, s] = top
        p["k"] = csa_inputs.f32_to_bf16_bits(k)
        return p
    if case == "one_wave_heavy":      # 100 planted keys all in one scan wave's keys: that wave's bound
        # sits far above the others' and one select segment holds them.  With 1024- or 2048-key scan
        # chunks of four waves, wave 0 of chunk 0 scores keys 128 j + i (i < 32, j < 8 or 16).
        p = csa_inputs.make_decode(B=3, context=4 * 32768, topk=2048, n_planted=100, seed=58)
        k = _bf16_to_f32(p["k"])
        mine = np.array([128 * j + i for j in range(16) for i in range(32)])[:100]
        for b in range(p["B"]):
            planted = k[b, int(p["planted"][b, 0])].copy()
            k[b, p["planted"][b]] = k[b, (p["planted"][b] + 1) % p["T"]]   # undo the spread plant
            k[b, mine] = planted
            p["planted"][b] = mine
        p["k"] = csa_inputs.f32_to_bf16_bits(k)
        return p
    if case == "odd_T":               # T and the visible counts not multiples of 4: score rows padded
        # to a multiple of 4 floats, 16-byte select loads over a partial last group, clamped key rows
        p = csa_inputs.make_decode(B=3, context=4 * 4099, topk=512, n_planted=8, seed=59)
        p["kv_len"] = np.array([4099, 4097, 2051], dtype=np.int32)
        return p
    if case == "noncausal":           # every key visible to every row, kv_len caps one sequence
        p = csa_inputs.make_decode(B=3, context=4 * 6000, topk=700, n_planted=8, S_q=4, seed=57)
        p["causal"] = False
        p["q_pos0"] = 0                                  # causal rows would see almost nothing
        p["kv_len"] = np.array([6000, 2500, 650], dtype=np.int32)
        return p
    raise ValueError(case)


@pytest.mark.parametrize("case", ["no_planted", "long_rows", "ragged_kv", "k_near_vis", "crowded_bin",
                                  "one_wave_heavy", "odd_T", "noncausal"])
@pytest.mark.parametrize("chunk", [0, 2048])
def test_decode_select_paths(case, chunk):
    """Each case with the default scan chunks and with 2048-key chunks forced
    (the small cases otherwise take 1024-key chunks)."""
    p = _select_case(case)
    _say(f"decode select path case {case} chunk={chunk}: B={p['B']} S_q={p['S_q']} T={p['T']} k={p['topk']}")
    with L.test_options(decode_chunk=chunk):
        idx, sc = _decode(p, return_scores=True)
    check_tolerance(p, np.arange(p["S_q"]), idx, sc, p["topk"])
    ref = _prefill(p)
    for b in range(p["B"]):
        for r in range(p["S_q"]):
            assert sorted(idx[b, r].tolist()) == sorted(ref[b, r].tolist()), f"row ({b},{r}) differs from prefill"
    if case == "one_wave_heavy":
        for b in range(p["B"]):
            assert set(p["planted"][b].tolist()) <= set(idx[b, 0].tolist())
    if case == "crowded_bin":         # ties among the rest: the lowest indices win
        for b in range(p["B"]):
            s = int(p["planted"][b, 0])
            want = [s] + [j for j in range(p["topk"]) if j != s][: p["topk"] - 1]
            assert sorted(idx[b, 0].tolist()) == sorted(want)
            assert (sc[b, 0] == sc[b, 0][idx[b, 0] != s][0]).sum() == p["topk"] - 1


def test_decode_all_scores_equal():
    """Every key identical: all scores tie, so the lowest indices win."""
    p = csa_inputs.make_decode(B=2, context=4 * 5000, topk=300, n_planted=0, seed=56)
    p["k"] = np.ascontiguousarray(np.repeat(p["k"][:, :1, :], p["T"], axis=1))
    _say("decode all-equal scores")
    idx, sc = _decode(p, return_scores=True)
    for b in range(p["B"]):
        assert sorted(idx[b, 0].tolist()) == list(range(p["topk"]))
        assert (sc[b, 0] == sc[b, 0, 0]).all()


def test_decode_long_chunks_exact_with_ragged_rows():
    """32 rows against T=32768 with k=2048 take the 2048-key scan chunks; with
    kv_len some rows are shorter than 8k (their waves cannot vouch for a tight
    bound, so the select runs over the dense scores), some end inside a chunk.
    Integer inputs: sets and scores must equal the oracle's exactly."""
    p = _integer_decode(B=16, S_q=2, T=32768, topk=2048, seed=61)
    p["kv_len"] = np.array([32768, 5000, 20000, 16384, 16383, 2047, 30001, 8192,
                            32768, 12345, 24576, 4097, 32000, 2049, 18000, 32767], dtype=np.int32)
    _say("decode long chunks: B=16 S_q=2 T=32768 k=2048, ragged kv_len")
    ref_i, ref_s, _ = oracle.oracle_topk(p)
    idx, sc = _decode(p, return_scores=True)
    check_exact(idx, ref_i, sc, ref_s)


def test_decode_chunk_sizes_same_sets():
    """The decode scan split into 1024-key and into 2048-key workgroup chunks
    gives the same sets and bitwise the same scores on one input (the config-4
    decode shape, all 32 rows), and integer inputs match the oracle exactly at
    both chunk sizes."""
    p = csa_inputs.config(4)
    _say("decode chunk invariance: config 4 with 1024- and 2048-key chunks")
    with L.test_options(decode_chunk=1024):
        a, sa = _decode(p, return_scores=True)
    with L.test_options(decode_chunk=2048):
        b, sb = _decode(p, return_scores=True)
    for bb in range(p["B"]):
        ma = dict(zip(a[bb, 0].tolist(), sa[bb, 0].view(np.uint32).tolist()))
        mb = dict(zip(b[bb, 0].tolist(), sb[bb, 0].view(np.uint32).tolist()))
        assert ma == mb, f"sequence {bb}: chunk sizes disagree"
    q = _integer_decode(B=4, S_q=2, T=20000, topk=1000, seed=71)
    ref_i, ref_s, _ = oracle.oracle_topk(q)
    for ch in (1024, 2048):
        with L.test_options(decode_chunk=ch):
            idx, sc = _decode(q, return_scores=True)
        check_exact(idx, ref_i, sc, ref_s)
