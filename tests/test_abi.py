"""C-ABI checks that need no GPU: exported symbols, argument validation
(which returns before any device work), workspace sizing, status strings,
and the host-side work counts used by the bench."""
import ctypes
import json
import os
import subprocess

import pytest

import lightning_indexer_top_02_amd as L
from lightning_indexer_top_02_amd import _binding as Bd
from lightning_indexer_top_02_amd import roofline as R

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa_indexer.h")


@pytest.fixture(scope="module")
def lib():
    return L.load_library()


def _declared_functions():
    import re
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:csa_status|const char\*|int)\s+(csa_\w+)\s*\(", text, re.M)))


def test_header_declares_and_library_exports_everything(lib):
    names = _declared_functions()
    assert names == sorted(Bd.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True, text=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    for n in names:
        assert n in exported, n
        assert hasattr(lib, n)


def test_struct_layout_matches_header():
    # uint32 + 7*int32 = 32 bytes, then int64 at 32, four pointers: 72 bytes
    assert ctypes.sizeof(Bd.CsaProblem) == 72
    assert Bd.CsaProblem.q_pos0.offset == 32
    assert Bd.CsaProblem.kv_len.offset == 64


def test_status_strings_and_version(lib):
    for s in range(5):
        assert lib.csa_status_str(s).decode().startswith("CSA_")
    assert b"unknown" in lib.csa_status_str(99)
    assert L.version() == 100


def _prob(**kw):
    p = Bd.CsaProblem()
    p.struct_size = ctypes.sizeof(Bd.CsaProblem)
    p.dtype = Bd.CSA_BF16
    p.B, p.S_q, p.T, p.H, p.D, p.m, p.q_pos0 = 1, 64, 256, 64, 128, 4, 0
    p.q, p.k, p.w = 0x1000, 0x2000, 0x3000     # never dereferenced on the error paths
    p.kv_len = None
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def _call_prefill(lib, p, topk=16, flags=0, out=0x4000, ws=None, ws_bytes=0):
    return lib.csa_index_topk_prefill(ctypes.byref(p) if p is not None else None, topk, flags,
                                      out, None, ws, ws_bytes, None)


@pytest.mark.parametrize("field,value,status", [
    ("struct_size", 8, Bd.CSA_ERR_INVALID),
    ("dtype", 7, Bd.CSA_ERR_INVALID),
    ("B", 0, Bd.CSA_ERR_INVALID),
    ("S_q", -1, Bd.CSA_ERR_INVALID),
    ("T", 0, Bd.CSA_ERR_INVALID),
    ("H", 0, Bd.CSA_ERR_INVALID),
    ("m", 0, Bd.CSA_ERR_INVALID),
    ("q_pos0", -5, Bd.CSA_ERR_INVALID),
    ("q", None, Bd.CSA_ERR_INVALID),
    ("k", None, Bd.CSA_ERR_INVALID),
    ("w", None, Bd.CSA_ERR_INVALID),
    ("D", 48, Bd.CSA_ERR_UNSUPPORTED),
    ("H", 129, Bd.CSA_ERR_UNSUPPORTED),
])
def test_problem_validation(lib, field, value, status):
    p = _prob(**{field: value})
    assert _call_prefill(lib, p) == status
    assert lib.csa_last_error().decode()


def test_other_argument_errors(lib):
    p = _prob()
    assert _call_prefill(lib, None) == Bd.CSA_ERR_INVALID
    assert _call_prefill(lib, p, topk=0) == Bd.CSA_ERR_INVALID
    assert _call_prefill(lib, p, topk=Bd.MAX_TOPK + 1) == Bd.CSA_ERR_UNSUPPORTED
    assert _call_prefill(lib, p, flags=8) == Bd.CSA_ERR_INVALID
    assert _call_prefill(lib, p, out=None) == Bd.CSA_ERR_INVALID
    # workspace too small -> rejected before anything is enqueued
    assert _call_prefill(lib, p, ws=0x5000, ws_bytes=16) == Bd.CSA_ERR_WORKSPACE
    # workspace not 16-byte aligned -> rejected before anything is enqueued
    assert _call_prefill(lib, p, ws=0x5004, ws_bytes=1 << 40) == Bd.CSA_ERR_INVALID
    # decode: too many query rows
    p2 = _prob(S_q=17)
    assert lib.csa_index_topk_decode(ctypes.byref(p2), 16, 0, 0x4000, None, None, 0, None) == Bd.CSA_ERR_UNSUPPORTED
    # threshold: tau outside (0,1), NaN bias, missing count
    for tau, bias, cnt in [(0.0, 0.0, 0x6000), (1.0, 0.0, 0x6000), (float("nan"), 0.0, 0x6000),
                           (0.5, float("inf"), 0x6000), (0.5, 0.0, None)]:
        assert lib.csa_index_threshold_select(ctypes.byref(p), tau, bias, 16, 0, 0x4000, cnt, None,
                                              None, 0, None) == Bd.CSA_ERR_INVALID
    # interleaved: P < 1, k_local < 1
    assert lib.csa_index_topk_interleaved(ctypes.byref(p), 0, 8, 0, 0x4000, None, None, 0, None) == Bd.CSA_ERR_INVALID
    assert lib.csa_index_topk_interleaved(ctypes.byref(p), 4, 0, 0, 0x4000, None, None, 0, None) == Bd.CSA_ERR_INVALID
    # recall
    assert lib.csa_set_recall(0x1, 0, 0x2, 4, 1, 10, 0x3, None, 0, None) == Bd.CSA_ERR_INVALID
    assert lib.csa_set_recall(0x1, 4, 0x2, 9000, 1, 10, 0x3, None, 0, None) == Bd.CSA_ERR_UNSUPPORTED
    assert lib.csa_set_recall(0x1, 4, 0x2, 4, -1, 10, 0x3, None, 0, None) == Bd.CSA_ERR_INVALID


def test_workspace_size(lib):
    p = _prob(S_q=4096, T=1024)
    sizes = {}
    for op in (Bd.OP_PREFILL, Bd.OP_THRESHOLD, Bd.OP_INTERLEAVED, Bd.OP_RECALL):
        sizes[op] = Bd.workspace_size(op, p if op != Bd.OP_RECALL else None, 256, 4, 0)
    with pytest.raises(Bd.CsaError):
        Bd.workspace_size(Bd.OP_DECODE, p, 256)          # decode takes at most 16 query rows
    assert sizes[Bd.OP_RECALL] == 0
    assert all(sizes[o] > 0 for o in (Bd.OP_PREFILL, Bd.OP_THRESHOLD, Bd.OP_INTERLEAVED))
    # monotone in k and in the number of query rows; sorting adds scratch
    a = Bd.workspace_size(Bd.OP_PREFILL, _prob(S_q=64), 64)
    b = Bd.workspace_size(Bd.OP_PREFILL, _prob(S_q=64), 512)
    c = Bd.workspace_size(Bd.OP_PREFILL, _prob(S_q=4096), 512)
    d = Bd.workspace_size(Bd.OP_PREFILL, _prob(S_q=4096), 512, 1, Bd.CSA_SORTED)
    assert a < b < c < d
    # decode workspace holds one fp32 score per (row, key)
    dd = Bd.workspace_size(Bd.OP_DECODE, _prob(B=32, S_q=1, T=32768), 2048)
    assert dd >= 32 * 32768 * 4
    # bounded: far below the materialised [B,S,H,T] fp32 tensor at the long-prefill shape
    big = Bd.workspace_size(Bd.OP_PREFILL, _prob(S_q=65536, T=16384), 2048)
    assert big < R.materialised_score_bytes(1, 65536, 64, 16384) / 256
    with pytest.raises(Bd.CsaError):
        Bd.workspace_size(99, p, 16)


def test_work_counts_match_page_sizes():
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "streamindex_sizes.json")))
    S, H, m = g["S"], g["H_I"], g["m"]
    nbytes = R.materialised_score_bytes(g["B"], S, H, S // m)
    # the page's "256 GB" is 2^38 bytes (256 GiB)
    assert nbytes == 2 ** 38 and nbytes / 2 ** 30 == g["stated_size_GB"]
    # 32x regime extension: the largest materialisable S was 1M/32
    assert g["stated_max_S_streaming"] // g["stated_regime_extension"] == 32768
    # needed and all-visible pairs (closed form: row t sees floor(t/4)+1 keys)
    need, allv = R.visible_pairs(16384, 0, 4, 4096, 2048)
    assert allv == sum(min(t // 4 + 1, 4096) for t in range(16384)) == 33562624
    assert need == 25169920
    assert R.prefill_flops(64, 128, need) == 412383969280
    assert R.decode_bytes(32, 1, 32768, 64, 128, 2048) == 269230080


def _attn_prob(**kw):
    p = Bd.CsaAttnProblem()
    p.struct_size = ctypes.sizeof(Bd.CsaAttnProblem)
    p.B, p.S_q, p.T, p.H, p.Dk, p.Dv = 32, 1, 32768, 64, 128, 128
    p.q, p.k, p.v = 0x1000, 0x2000, 0x3000      # never dereferenced on the error paths
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def test_attention_struct_layout():
    # uint32 + 6*int32 = 28 bytes, pointers from 32: 56 bytes
    assert ctypes.sizeof(Bd.CsaAttnProblem) == 56
    assert Bd.CsaAttnProblem.q.offset == 32


def test_attention_workspace_size(lib):
    n = ctypes.c_size_t(0)
    # 32 rows, 8 chunks of 256 entries -> 8 workgroups per row
    assert lib.csa_attention_workspace_size(ctypes.byref(_attn_prob()), 2048, ctypes.byref(n)) == 0
    assert n.value == 32 * 8 * 64 * 128 * 4 + 2 * (32 * 8 * 64 * 4)
    # many rows: one workgroup per row
    assert lib.csa_attention_workspace_size(ctypes.byref(_attn_prob(B=4, S_q=512)), 2048, ctypes.byref(n)) == 0
    assert n.value == 2048 * 64 * 128 * 4 + 2 * (2048 * 64 * 4)


def test_attention_argument_errors(lib):
    def call(p, idx=0x5000, n_sel=2048, scale=0.1, out=0x6000, ws=0x7000, ws_bytes=1 << 40):
        return lib.csa_sparse_attention(ctypes.byref(p) if p is not None else None, idx, n_sel, scale, out, ws,
                                        ws_bytes, None)
    assert call(None) == Bd.CSA_ERR_INVALID
    assert call(_attn_prob(struct_size=8)) == Bd.CSA_ERR_INVALID
    assert call(_attn_prob(H=32)) == Bd.CSA_ERR_UNSUPPORTED
    assert call(_attn_prob(Dv=64)) == Bd.CSA_ERR_UNSUPPORTED
    assert call(_attn_prob(T=0)) == Bd.CSA_ERR_INVALID
    assert call(_attn_prob(), n_sel=0) == Bd.CSA_ERR_INVALID
    assert call(_attn_prob(), idx=None) == Bd.CSA_ERR_INVALID
    assert call(_attn_prob(), out=None) == Bd.CSA_ERR_INVALID
    assert call(_attn_prob(), scale=float("nan")) == Bd.CSA_ERR_INVALID
    assert call(_attn_prob(), ws_bytes=16) == Bd.CSA_ERR_WORKSPACE
    assert call(_attn_prob(), ws=0x7004) == Bd.CSA_ERR_INVALID


def test_union_argument_errors(lib):
    P = ctypes.c_void_p * 2
    W = ctypes.c_int32 * 2

    def call(L=2, rows=4, T=100, cap=8, lists=(0x1000, 0x2000), widths=(4, 4), out=0x3000):
        return lib.csa_union_rows(P(*lists), W(*widths), L, rows, T, cap, out, None, None)
    assert call(L=0) == Bd.CSA_ERR_INVALID
    assert call(L=9) == Bd.CSA_ERR_INVALID
    assert call(rows=-1) == Bd.CSA_ERR_INVALID
    assert call(T=0) == Bd.CSA_ERR_INVALID
    assert call(cap=0) == Bd.CSA_ERR_INVALID
    assert call(T=(1 << 20) + 1) == Bd.CSA_ERR_UNSUPPORTED
    assert call(widths=(4, 0)) == Bd.CSA_ERR_INVALID
    assert call(lists=(0x1000, 0)) == Bd.CSA_ERR_INVALID
    assert call(out=None) == Bd.CSA_ERR_INVALID
    # one 1024-thread workgroup per row: a dispatch holds at most 2^32 work-items
    assert call(rows=1 << 22) == Bd.CSA_ERR_UNSUPPORTED
    assert lib.csa_set_recall(0x1000, 8, 0x2000, 8, 1 << 24, 100, 0x3000, None, 0, None) == Bd.CSA_ERR_UNSUPPORTED


def test_threshold_layers_argument_errors(lib):
    def call(probs, L=None, tau=0.5, cap=64, idx=None, cnt=None, ws=0x7000, ws_bytes=1 << 40):
        n = len(probs)
        PP = (ctypes.POINTER(Bd.CsaProblem) * max(n, 1))(*[ctypes.pointer(p) for p in probs])
        V = ctypes.c_void_p * max(n, 1)
        I = V(*(idx if idx is not None else [0x4000 + 0x100 * i for i in range(n)]))
        C = V(*(cnt if cnt is not None else [0x8000 + 0x100 * i for i in range(n)]))
        return lib.csa_index_threshold_select_layers(PP, n if L is None else L, tau, 0.0, cap, 0, I, C, None, ws,
                                                     ws_bytes, None)
    dec = lambda **kw: _prob(S_q=1, **kw)            # noqa: E731
    assert call([dec(), dec()], L=0) == Bd.CSA_ERR_INVALID
    assert call([dec()] * 9) == Bd.CSA_ERR_INVALID
    assert call([dec(), dec()], tau=1.0) == Bd.CSA_ERR_INVALID
    assert call([dec(), dec()], cap=0) == Bd.CSA_ERR_INVALID
    assert call([dec(), dec(B=0)]) == Bd.CSA_ERR_INVALID
    assert call([dec(), dec()], cnt=[0x8000, 0]) == Bd.CSA_ERR_INVALID
    assert call([dec(), _prob(S_q=17)]) == Bd.CSA_ERR_UNSUPPORTED      # not decode-shaped
    assert call([dec(), dec(T=300)]) == Bd.CSA_ERR_UNSUPPORTED         # shapes differ
    assert call([dec(), dec(B=2)]) == Bd.CSA_ERR_UNSUPPORTED
    assert call([dec(), dec()], ws_bytes=16) == Bd.CSA_ERR_WORKSPACE
    assert call([dec(), dec()], ws=0x7004) == Bd.CSA_ERR_INVALID
    # the workspace is the per-layer threshold workspace times the layer count
    n1 = L.workspace_size(L.OP_THRESHOLD, dec(), 64, 1, 0)
    assert call([dec(), dec(), dec()], ws_bytes=3 * n1 - 1) == Bd.CSA_ERR_WORKSPACE


def test_project_argument_errors(lib):
    def call(M=300, N=200, K=128, dt=Bd.CSA_BF16, x=0x1000, w=0x2000, y=0x3000):
        return lib.csa_project(x, w, M, N, K, dt, y, None)
    assert call(M=-1) == Bd.CSA_ERR_INVALID
    assert call(N=0) == Bd.CSA_ERR_INVALID
    assert call(K=0) == Bd.CSA_ERR_INVALID
    assert call(dt=7) == Bd.CSA_ERR_INVALID
    assert call(K=100) == Bd.CSA_ERR_UNSUPPORTED                    # K must be a multiple of 64
    assert call(N=(1 << 20) + 1) == Bd.CSA_ERR_UNSUPPORTED
    assert call(M=1 << 31) == Bd.CSA_ERR_UNSUPPORTED
    assert call(x=None) == Bd.CSA_ERR_INVALID
    assert call(y=None) == Bd.CSA_ERR_INVALID
    assert call(x=0x1008) == Bd.CSA_ERR_INVALID                     # 16-byte alignment
    assert call(dt=Bd.CSA_F32, y=0x3002) == Bd.CSA_ERR_INVALID
    assert call(M=0, x=None, w=None, y=None) == Bd.CSA_OK           # nothing to do


def test_test_options(lib):
    """csa_set_test_option: valid values accepted, others rejected with the
    option unchanged; the binding's context manager resets to 0."""
    for opt, good, bad in [(Bd.CSA_OPT_FORCE_GENERIC, [0, 1], [2, -1]),
                           (Bd.CSA_OPT_CAND_CAP, [0, 1, 1 << 20], [-1, (1 << 30) + 1]),
                           (Bd.CSA_OPT_DECODE_CHUNK, [0, 1024, 2048], [512, 4096, 1])]:
        for v in good:
            assert lib.csa_set_test_option(opt, v) == Bd.CSA_OK
        for v in bad:
            assert lib.csa_set_test_option(opt, v) == Bd.CSA_ERR_INVALID
            assert lib.csa_last_error().decode()
        assert lib.csa_set_test_option(opt, 0) == Bd.CSA_OK
    assert lib.csa_set_test_option(99, 0) == Bd.CSA_ERR_INVALID
    p = _prob(S_q=256)
    base = Bd.workspace_size(Bd.OP_PREFILL, p, 64)
    with L.test_options(cand_cap=4096):                  # larger candidate buffers need more workspace
        assert Bd.workspace_size(Bd.OP_PREFILL, p, 64) > base
    assert Bd.workspace_size(Bd.OP_PREFILL, p, 64) == base
    with pytest.raises(ValueError):
        L.test_options(no_such_option=1)


def test_prefill_size_limits_reject_before_enqueue(lib):
    """Work the kernels cannot index is refused with CSA_ERR_UNSUPPORTED before
    anything is enqueued (the pointers here are never dereferenced)."""
    # B * ceil(S_q / 4) * P query blocks above what one launch counts in 32 bits
    p = _prob(S_q=1 << 30, T=1 << 20)
    assert lib.csa_index_topk_interleaved(ctypes.byref(p), 16, 1, 0, 0x4000, None, 0x5000, 1 << 60,
                                          None) == Bd.CSA_ERR_UNSUPPORTED
    assert "query blocks" in lib.csa_last_error().decode()
    # CSA_SORTED launches one sort workgroup per output row segment (B * S_q * P)
    p = _prob(S_q=1 << 22, T=1 << 20)
    assert lib.csa_index_topk_interleaved(ctypes.byref(p), 8, 1, Bd.CSA_SORTED, 0x4000, None, 0x5000, 1 << 60,
                                          None) == Bd.CSA_ERR_UNSUPPORTED
    assert "CSA_SORTED" in lib.csa_last_error().decode()
