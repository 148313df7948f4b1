"""ctypes binding of libcsa_indexer.so.

Argument marshalling only: every step of the indexer runs in the library's
HIP kernels.  Tensors are torch tensors on the current HIP device; outputs
and workspace are allocated with torch (or passed in), and every call is
enqueued on torch's current stream.  The library must be built
(``python -m lightning_indexer_top_02_amd.build``); there is no fallback.
"""
from __future__ import annotations

import ctypes
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcsa_indexer.so")

CSA_OK, CSA_ERR_INVALID, CSA_ERR_UNSUPPORTED, CSA_ERR_WORKSPACE, CSA_ERR_DEVICE = range(5)
CSA_BF16, CSA_F32 = 0, 1
CSA_SORTED, CSA_NONCAUSAL = 1, 2
OP_PREFILL, OP_DECODE, OP_THRESHOLD, OP_INTERLEAVED, OP_RECALL = range(5)
MAX_TOPK = 4096
MAX_DECODE_SQ = 16


class CsaError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{message} (status {status})")
        self.status = status


class CsaProblem(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("dtype", ctypes.c_int32),
        ("B", ctypes.c_int32), ("S_q", ctypes.c_int32), ("T", ctypes.c_int32),
        ("H", ctypes.c_int32), ("D", ctypes.c_int32),
        ("m", ctypes.c_int32),
        ("q_pos0", ctypes.c_int64),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("w", ctypes.c_void_p),
        ("kv_len", ctypes.c_void_p),
    ]


class CsaAttnProblem(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("B", ctypes.c_int32), ("S_q", ctypes.c_int32), ("T", ctypes.c_int32),
        ("H", ctypes.c_int32), ("Dk", ctypes.c_int32), ("Dv", ctypes.c_int32),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
    ]


_P = ctypes.POINTER(CsaProblem)
_PA = ctypes.POINTER(CsaAttnProblem)
_vp, _i32, _u32, _f32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_float, ctypes.c_size_t

_SIGS = {
    "csa_workspace_size": (_i32, [ctypes.c_int, _P, _i32, _i32, _u32, ctypes.POINTER(_sz)]),
    "csa_index_topk_prefill": (_i32, [_P, _i32, _u32, _vp, _vp, _vp, _sz, _vp]),
    "csa_index_topk_decode": (_i32, [_P, _i32, _u32, _vp, _vp, _vp, _sz, _vp]),
    "csa_index_topk_decode_noalloc": (_i32, [_P, _i32, _u32, _vp, _vp, _vp]),
    "csa_index_threshold_select": (_i32, [_P, _f32, _f32, _i32, _u32, _vp, _vp, _vp, _vp, _sz, _vp]),
    "csa_index_threshold_select_layers": (_i32, [ctypes.POINTER(_P), _i32, _f32, _f32, _i32, _u32,
                                                 ctypes.POINTER(_vp), ctypes.POINTER(_vp), ctypes.POINTER(_vp),
                                                 _vp, _sz, _vp]),
    "csa_index_topk_interleaved": (_i32, [_P, _i32, _i32, _u32, _vp, _vp, _vp, _sz, _vp]),
    "csa_set_recall": (_i32, [_vp, _i32, _vp, _i32, ctypes.c_int64, _i32, _vp, _vp, _sz, _vp]),
    "csa_attention_workspace_size": (_i32, [_PA, _i32, ctypes.POINTER(_sz)]),
    "csa_sparse_attention": (_i32, [_PA, _vp, _i32, _f32, _vp, _vp, _sz, _vp]),
    "csa_union_rows": (_i32, [ctypes.POINTER(_vp), ctypes.POINTER(_i32), _i32, ctypes.c_int64, _i32, _i32, _vp,
                              _vp, _vp]),
    "csa_project": (_i32, [_vp, _vp, ctypes.c_int64, _i32, _i32, _i32, _vp, _vp]),
    "csa_set_test_option": (_i32, [_i32, ctypes.c_int64]),
    "csa_status_str": (ctypes.c_char_p, [_i32]),
    "csa_last_error": (ctypes.c_char_p, []),
    "csa_version": (ctypes.c_int, []),
}

EXPORTS = tuple(_SIGS)

_lib = None


def load_library(path: str = LIB_PATH):
    """Load the shared library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m lightning_indexer_top_02_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status):
    if status != CSA_OK:
        lib = load_library()
        raise CsaError(status, lib.csa_last_error().decode() or lib.csa_status_str(status).decode())


def version() -> int:
    return load_library().csa_version()


CSA_OPT_FORCE_GENERIC, CSA_OPT_CAND_CAP, CSA_OPT_DECODE_CHUNK = 1, 2, 3
_TEST_OPTIONS = {"force_generic": CSA_OPT_FORCE_GENERIC, "cand_cap": CSA_OPT_CAND_CAP,
                 "decode_chunk": CSA_OPT_DECODE_CHUNK}


class test_options:
    """Context manager over csa_set_test_option: e.g.
    ``with test_options(cand_cap=1): ...`` forces the prefill kernels to
    compact their candidate lists on almost every key tile; the options go
    back to 0 (automatic) on exit.  For tests: the options change which
    kernel variant runs, never the results."""

    __test__ = False                                   # not a pytest class

    def __init__(self, **opts):
        unknown = set(opts) - set(_TEST_OPTIONS)
        if unknown:
            raise ValueError(f"unknown test options {sorted(unknown)}")
        self.opts = opts

    def __enter__(self):
        lib = load_library()
        for name, val in self.opts.items():
            _check(lib.csa_set_test_option(_TEST_OPTIONS[name], int(val)))
        return self

    def __exit__(self, *exc):
        lib = load_library()
        for name in self.opts:
            lib.csa_set_test_option(_TEST_OPTIONS[name], 0)
        return False


# ---------------------------------------------------------------------------
# torch plumbing


def _torch():
    import torch
    return torch


def _stream_handle():
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def make_problem(q, k, w, m=4, q_pos0=0, kv_len=None):
    """Check tensors and build the C problem struct (keeps the tensors alive)."""
    torch = _torch()
    if q.dim() != 4 or k.dim() != 3 or w.dim() != 3:
        raise ValueError("expected q [B,S_q,H,D], k [B,T,D], w [B,S_q,H]")
    B, S_q, H, D = q.shape
    if k.shape[0] != B or k.shape[2] != D or tuple(w.shape) != (B, S_q, H):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)} k {tuple(k.shape)} w {tuple(w.shape)}")
    if q.dtype != k.dtype or q.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("q and k must share dtype bfloat16 or float32")
    if w.dtype != torch.float32:
        raise TypeError("w must be float32")
    for name, t in (("q", q), ("k", k), ("w", w)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if kv_len is not None:
        if kv_len.dtype != torch.int32 or not kv_len.is_cuda or kv_len.numel() != B or not kv_len.is_contiguous():
            raise ValueError("kv_len must be a contiguous int32 GPU tensor of B entries")
    p = CsaProblem()
    p.struct_size = ctypes.sizeof(CsaProblem)
    p.dtype = CSA_BF16 if q.dtype == torch.bfloat16 else CSA_F32
    p.B, p.S_q, p.T, p.H, p.D = B, S_q, k.shape[1], H, D
    p.m = int(m)
    p.q_pos0 = int(q_pos0)
    p.q, p.k, p.w = q.data_ptr(), k.data_ptr(), w.data_ptr()
    p.kv_len = None if kv_len is None else kv_len.data_ptr()
    return p


def _flags(sorted_, causal):
    return (CSA_SORTED if sorted_ else 0) | (0 if causal else CSA_NONCAUSAL)


def workspace_size(op, prob, k_or_cap, P=1, flags=0) -> int:
    n = _sz(0)
    _check(load_library().csa_workspace_size(op, ctypes.byref(prob) if prob is not None else None,
                                             int(k_or_cap), int(P), int(flags), ctypes.byref(n)))
    return n.value


def _workspace(nbytes, device, ws=None):
    torch = _torch()
    if nbytes == 0:
        return None
    if ws is not None:
        if ws.numel() * ws.element_size() < nbytes:
            raise ValueError(f"workspace has {ws.numel() * ws.element_size()} bytes, needs {nbytes}")
        return ws
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def index_topk_prefill(q, k, w, topk, *, m=4, q_pos0=0, kv_len=None, sorted=False, causal=True,
                       return_scores=False, out=None, out_score=None, workspace=None):
    """Top-k key indices per query row: int32 [B, S_q, topk] (and fp32 scores)."""
    torch = _torch()
    prob = make_problem(q, k, w, m, q_pos0, kv_len)
    flags = _flags(sorted, causal)
    B, S_q = q.shape[0], q.shape[1]
    idx = out if out is not None else torch.empty((B, S_q, topk), dtype=torch.int32, device=q.device)
    sc = out_score if out_score is not None else (
        torch.empty((B, S_q, topk), dtype=torch.float32, device=q.device) if return_scores else None)
    ws = _workspace(workspace_size(OP_PREFILL, prob, topk, 1, flags), q.device, workspace)
    _check(load_library().csa_index_topk_prefill(ctypes.byref(prob), int(topk), flags, _ptr(idx), _ptr(sc),
                                                 _ptr(ws), _nbytes(ws), _stream_handle()))
    return (idx, sc) if sc is not None else idx


def index_topk_decode(q, k, w, topk, *, m=4, q_pos0=0, kv_len=None, sorted=False, causal=True,
                      return_scores=False, out=None, out_score=None, workspace=None):
    """Decode-shaped top-k (S_q <= 16): same result sets as index_topk_prefill."""
    torch = _torch()
    prob = make_problem(q, k, w, m, q_pos0, kv_len)
    flags = _flags(sorted, causal)
    B, S_q = q.shape[0], q.shape[1]
    idx = out if out is not None else torch.empty((B, S_q, topk), dtype=torch.int32, device=q.device)
    sc = out_score if out_score is not None else (
        torch.empty((B, S_q, topk), dtype=torch.float32, device=q.device) if return_scores else None)
    ws = _workspace(workspace_size(OP_DECODE, prob, topk, 1, flags), q.device, workspace)
    _check(load_library().csa_index_topk_decode(ctypes.byref(prob), int(topk), flags, _ptr(idx), _ptr(sc),
                                                _ptr(ws), _nbytes(ws), _stream_handle()))
    return (idx, sc) if sc is not None else idx


def index_topk_decode_noalloc(q, k, w, topk, *, m=4, q_pos0=0, kv_len=None, sorted=False, causal=True,
                              return_scores=False, out=None, out_score=None):
    """index_topk_decode that takes no workspace: the library uses its fixed
    per-GPU scratch (NOALLOC_SCRATCH_BYTES).  Calls that overlap on one GPU
    race; calls on one stream are safe."""
    torch = _torch()
    prob = make_problem(q, k, w, m, q_pos0, kv_len)
    B, S_q = q.shape[0], q.shape[1]
    idx = out if out is not None else torch.empty((B, S_q, topk), dtype=torch.int32, device=q.device)
    sc = out_score if out_score is not None else (
        torch.empty((B, S_q, topk), dtype=torch.float32, device=q.device) if return_scores else None)
    _check(load_library().csa_index_topk_decode_noalloc(ctypes.byref(prob), int(topk), _flags(sorted, causal),
                                                        _ptr(idx), _ptr(sc), _stream_handle()))
    return (idx, sc) if sc is not None else idx


NOALLOC_SCRATCH_BYTES = 8 << 20


def index_threshold_select(q, k, w, cap, *, prob_threshold=0.5, logit_bias=0.0, m=4, q_pos0=0, kv_len=None,
                           sorted=False, causal=True, return_scores=False, workspace=None):
    """Keys with sigmoid(I + bias) > prob_threshold: (idx [B,S_q,cap], count [B,S_q][, scores])."""
    torch = _torch()
    prob = make_problem(q, k, w, m, q_pos0, kv_len)
    flags = _flags(sorted, causal)
    B, S_q = q.shape[0], q.shape[1]
    idx = torch.empty((B, S_q, cap), dtype=torch.int32, device=q.device)
    cnt = torch.empty((B, S_q), dtype=torch.int32, device=q.device)
    sc = torch.empty((B, S_q, cap), dtype=torch.float32, device=q.device) if return_scores else None
    ws = _workspace(workspace_size(OP_THRESHOLD, prob, cap, 1, flags), q.device, workspace)
    _check(load_library().csa_index_threshold_select(ctypes.byref(prob), float(prob_threshold), float(logit_bias),
                                                     int(cap), flags, _ptr(idx), _ptr(cnt), _ptr(sc), _ptr(ws),
                                                     _nbytes(ws), _stream_handle()))
    return (idx, cnt, sc) if sc is not None else (idx, cnt)


MAX_LAYERS = 8


def batchable_layers(layers) -> bool:
    """True when index_threshold_select_layers takes these (q, k, w) layers:
    at most MAX_LAYERS, all bf16 with H=64, D=128, S_q <= MAX_DECODE_SQ, and
    the same B, S_q and T."""
    torch = _torch()
    if not 1 <= len(layers) <= MAX_LAYERS:
        return False
    q0, k0, _ = layers[0]
    for q, k, w in layers:
        if q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16:
            return False
        if q.dim() != 4 or k.dim() != 3 or q.shape[2] != 64 or q.shape[3] != 128 or q.shape[1] > MAX_DECODE_SQ:
            return False
        if q.shape[:2] != q0.shape[:2] or k.shape[1] != k0.shape[1]:
            return False
    return True


def index_threshold_select_layers(layers, cap, *, prob_threshold=0.5, logit_bias=0.0, m=4, q_pos0=0, kv_len=None,
                                  sorted=False, causal=True, workspace=None):
    """index_threshold_select over several same-shape decode problems
    (layers: sequence of (q, k, w)) in one launch per kernel; returns a list
    of (idx [B,S_q,cap], count [B,S_q]), one per layer."""
    torch = _torch()
    if not batchable_layers(layers):
        raise ValueError("layers must be 1..8 bf16 decode problems (H=64, D=128, S_q<=16) of one shape")
    probs = [make_problem(q, k, w, m, q_pos0, kv_len) for q, k, w in layers]
    flags = _flags(sorted, causal)
    B, S_q = layers[0][0].shape[:2]
    dev = layers[0][0].device
    idx = [torch.empty((B, S_q, cap), dtype=torch.int32, device=dev) for _ in layers]
    cnt = [torch.empty((B, S_q), dtype=torch.int32, device=dev) for _ in layers]
    n = len(layers)
    ws = _workspace(n * workspace_size(OP_THRESHOLD, probs[0], cap, 1, flags), dev, workspace)
    pp = (_P * n)(*[ctypes.pointer(p) for p in probs])
    pi = (_vp * n)(*[_ptr(t) for t in idx])
    pc = (_vp * n)(*[_ptr(t) for t in cnt])
    _check(load_library().csa_index_threshold_select_layers(pp, n, float(prob_threshold), float(logit_bias),
                                                            int(cap), flags, pi, pc, None, _ptr(ws), _nbytes(ws),
                                                            _stream_handle()))
    return list(zip(idx, cnt))


def index_topk_interleaved(q, k, w, P, k_local, *, m=4, q_pos0=0, kv_len=None, sorted=False, causal=True,
                           return_scores=False, out=None, workspace=None):
    """Per-partition (s mod P) local top-k_local: int32 [B, S_q, P*k_local]."""
    torch = _torch()
    prob = make_problem(q, k, w, m, q_pos0, kv_len)
    flags = _flags(sorted, causal)
    B, S_q = q.shape[0], q.shape[1]
    idx = out if out is not None else torch.empty((B, S_q, P * k_local), dtype=torch.int32, device=q.device)
    sc = torch.empty((B, S_q, P * k_local), dtype=torch.float32, device=q.device) if return_scores else None
    ws = _workspace(workspace_size(OP_INTERLEAVED, prob, k_local, P, flags), q.device, workspace)
    _check(load_library().csa_index_topk_interleaved(ctypes.byref(prob), int(P), int(k_local), flags, _ptr(idx),
                                                     _ptr(sc), _ptr(ws), _nbytes(ws), _stream_handle()))
    return (idx, sc) if sc is not None else idx


def set_recall(sel, ref, T, out=None):
    """Per-row |set(sel) ∩ set(ref)| / |set(ref)| (entries < 0 ignored) as fp32 [rows]."""
    torch = _torch()
    if sel.dtype != torch.int32 or ref.dtype != torch.int32:
        raise TypeError("sel and ref must be int32")
    if not (sel.is_cuda and ref.is_cuda and sel.is_contiguous() and ref.is_contiguous()):
        raise ValueError("sel and ref must be contiguous GPU tensors")
    n_sel, n_ref = sel.shape[-1], ref.shape[-1]
    rows = sel.numel() // n_sel
    if ref.numel() // n_ref != rows:
        raise ValueError("sel and ref must have the same number of rows")
    rec = out if out is not None else torch.empty(rows, dtype=torch.float32, device=sel.device)
    _check(load_library().csa_set_recall(_ptr(sel), int(n_sel), _ptr(ref), int(n_ref), int(rows), int(T),
                                         _ptr(rec), None, 0, _stream_handle()))
    return rec


def make_attn_problem(q, k, v):
    """Describe bf16 q [B,S_q,H,Dk], k [B,T,Dk], v [B,T,Dv] (contiguous GPU tensors)."""
    torch = _torch()
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != torch.bfloat16:
            raise TypeError(f"{name} must be bfloat16")
        if not (t.is_cuda and t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    B, S_q, H, Dk = q.shape
    if k.shape[0] != B or v.shape[0] != B or k.shape[1] != v.shape[1] or k.shape[2] != Dk:
        raise ValueError("shape mismatch between q, k and v")
    return CsaAttnProblem(ctypes.sizeof(CsaAttnProblem), B, S_q, k.shape[1], H, Dk, v.shape[2],
                          _ptr(q), _ptr(k), _ptr(v))


def attention_workspace_size(prob, n_sel) -> int:
    n = _sz(0)
    _check(load_library().csa_attention_workspace_size(ctypes.byref(prob), int(n_sel), ctypes.byref(n)))
    return n.value


def sparse_attention(q, k, v, idx, *, scale=None, out=None, workspace=None):
    """Softmax attention of every head of q [B,S_q,H,Dk] over the key and value
    rows idx [B,S_q,n_sel] selects (entries outside [0, T) skipped); returns
    fp32 [B,S_q,H,Dv].  scale defaults to 1/sqrt(Dk)."""
    torch = _torch()
    if idx.dtype != torch.int32 or not (idx.is_cuda and idx.is_contiguous()):
        raise TypeError("idx must be a contiguous int32 GPU tensor")
    prob = make_attn_problem(q, k, v)
    n_sel = idx.shape[-1]
    if idx.numel() != q.shape[0] * q.shape[1] * n_sel:
        raise ValueError("idx must be [B, S_q, n_sel]")
    scale = float(1.0 / math.sqrt(q.shape[3])) if scale is None else float(scale)
    o = out if out is not None else torch.empty((q.shape[0], q.shape[1], q.shape[2], v.shape[2]),
                                               dtype=torch.float32, device=q.device)
    ws = _workspace(attention_workspace_size(prob, n_sel), q.device, workspace)
    _check(load_library().csa_sparse_attention(ctypes.byref(prob), _ptr(idx), int(n_sel), scale, _ptr(o),
                                               _ptr(ws), _nbytes(ws), _stream_handle()))
    return o


def union_rows(lists, T, cap, *, with_count=True):
    """Per-row union of index lists (each an int32 GPU tensor [..., width] with
    the same leading shape): ascending distinct indices in [0, T), -1 padded
    to `cap`; also the true union sizes (int32, leading shape) if with_count."""
    torch = _torch()
    if not lists:
        raise ValueError("need at least one list")
    lead = lists[0].shape[:-1]
    for t in lists:
        if t.dtype != torch.int32 or not (t.is_cuda and t.is_contiguous()):
            raise TypeError("lists must be contiguous int32 GPU tensors")
        if t.shape[:-1] != lead:
            raise ValueError("lists must share their leading shape")
    rows = 1
    for d in lead:
        rows *= int(d)
    ptrs = (_vp * len(lists))(*[_ptr(t) for t in lists])
    widths = (_i32 * len(lists))(*[int(t.shape[-1]) for t in lists])
    out = torch.empty(tuple(lead) + (int(cap),), dtype=torch.int32, device=lists[0].device)
    cnt = torch.empty(tuple(lead), dtype=torch.int32, device=lists[0].device) if with_count else None
    _check(load_library().csa_union_rows(ptrs, widths, len(lists), rows, int(T), int(cap), _ptr(out),
                                         _ptr(cnt) if cnt is not None else None, _stream_handle()))
    return (out, cnt) if with_count else out


class MultiLayerSelector:
    """OR-union of several indexer layers' threshold selections, recomputed
    every `tau` decode steps and reused in between (FlashMemory-DeepSeek-V4
    review: Memory Indexer on three layers, keep decisions OR-ed, a decode
    trigger interval of 64 steps).  Same-shape decode layers are selected in
    one batched launch (`batched=True`); otherwise each layer's selection runs
    in turn, or on its own HIP stream (`overlap=True`), joined before the
    union on the caller's current stream.  All compute is in the library's
    kernels."""

    def __init__(self, tau=64, prob_threshold=0.5, logit_bias=0.0, cap=2048, union_cap=None, overlap=False,
                 batched=True):
        self.tau = int(tau)
        self.prob_threshold = float(prob_threshold)
        self.logit_bias = float(logit_bias)
        self.cap = int(cap)
        self.union_cap = int(union_cap) if union_cap is not None else None
        self.overlap = bool(overlap)
        self.batched = bool(batched)
        self.refreshes = 0
        self._cached = None
        self._streams = []

    def select(self, step, layers, *, m=4, q_pos0=0, kv_len=None, causal=True):
        """layers: sequence of (q, k, w) indexer inputs, one per layer, sharing
        B, S_q and T.  Returns (union [B, S_q, union_cap], count [B, S_q])."""
        if self._cached is not None and step % self.tau != 0:
            return self._cached
        torch = _torch()
        T = layers[0][1].shape[1]
        ucap = self.union_cap if self.union_cap is not None else min(T, self.cap * len(layers))
        main = torch.cuda.current_stream()
        sels = []
        if self.batched and batchable_layers(layers):
            sels = [idx for idx, _ in index_threshold_select_layers(
                layers, self.cap, prob_threshold=self.prob_threshold, logit_bias=self.logit_bias, m=m,
                q_pos0=q_pos0, kv_len=kv_len, causal=causal)]
        elif self.overlap:
            while len(self._streams) < len(layers):      # created once, default priority
                self._streams.append(torch.cuda.Stream())
            streams = self._streams[: len(layers)]
            for s in streams:
                s.wait_stream(main)
            for (q, k, w), s in zip(layers, streams):
                with torch.cuda.stream(s):
                    idx, _ = index_threshold_select(q, k, w, self.cap, prob_threshold=self.prob_threshold,
                                                    logit_bias=self.logit_bias, m=m, q_pos0=q_pos0,
                                                    kv_len=kv_len, causal=causal)
                    sels.append(idx)
            for s, idx in zip(streams, sels):
                main.wait_stream(s)
                idx.record_stream(main)
        else:
            for q, k, w in layers:
                idx, _ = index_threshold_select(q, k, w, self.cap, prob_threshold=self.prob_threshold,
                                                logit_bias=self.logit_bias, m=m, q_pos0=q_pos0, kv_len=kv_len,
                                                causal=causal)
                sels.append(idx)
        self._cached = union_rows(sels, T, ucap)
        self.refreshes += 1
        return self._cached


def _topk_any(q, k, w, topk, **kw):
    """Top-k through the decode entry for decode-shaped rows, else prefill."""
    if q.shape[1] <= MAX_DECODE_SQ:
        return index_topk_decode(q, k, w, topk, **kw)
    return index_topk_prefill(q, k, w, topk, **kw)


class MultiLayerIndexer:
    """Previous-layer reuse across a stack of sparse-attention layers
    (Multi-layer Indexer post, "MLI"): layer l >= 1 attends to the top-k that
    layer l-1's indexer picked, while layer l's own indexer runs on a second
    HIP stream to serve layer l+1 (`overlap=True`); layer 0 runs its own
    indexer before its attention.  By default the same schedule is issued on
    the caller's stream alone (identical results): at B=32, T=32768 the scan
    fills every CU, so a concurrent attention only waits for it and the
    stream joins add time.  All compute is in the library's kernels."""

    def __init__(self, topk=2048, overlap=False):
        self.topk = int(topk)
        self.overlap = bool(overlap)
        self._side = None

    def run(self, layers, *, m=4, q_pos0=0, kv_len=None, causal=True, scale=None):
        """layers: sequence of ((q_I, k_I, w_I), (q, k, v)) per layer: the
        indexer's inputs and the attention's.  Returns the attention outputs,
        fp32 [B, S_q, H, Dv] per layer."""
        torch = _torch()
        kw = dict(m=m, q_pos0=q_pos0, kv_len=kv_len, causal=causal)
        main = torch.cuda.current_stream()
        if self.overlap and self._side is None:
            self._side = torch.cuda.Stream()              # created once, default priority
        sel = _topk_any(*layers[0][0], self.topk, **kw)
        outs = []
        for li, (ind, att) in enumerate(layers):
            nxt = None
            if 1 <= li < len(layers) - 1:                  # its result serves layer li+1
                if self.overlap:
                    self._side.wait_stream(main)
                    with torch.cuda.stream(self._side):
                        nxt = _topk_any(*ind, self.topk, **kw)
                else:
                    nxt = _topk_any(*ind, self.topk, **kw)
            outs.append(sparse_attention(*att, sel, scale=scale))
            if nxt is not None:
                if self.overlap:
                    main.wait_stream(self._side)
                    nxt.record_stream(main)
                sel = nxt
        return outs


def project(x, w, *, out_dtype=None, out=None):
    """y [..., N] = x [..., K] . w [N, K]^T (bf16 operands, fp32 accumulation);
    bf16 output unless out_dtype=torch.float32.  K must be a multiple of 64."""
    torch = _torch()
    out_dtype = torch.bfloat16 if out_dtype is None else out_dtype
    for name, t in (("x", x), ("w", w)):
        if t.dtype != torch.bfloat16:
            raise TypeError(f"{name} must be bfloat16")
        if not (t.is_cuda and t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    if w.dim() != 2 or x.shape[-1] != w.shape[1]:
        raise ValueError(f"shape mismatch: x {tuple(x.shape)} w {tuple(w.shape)}")
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out_dtype must be bfloat16 or float32")
    N, K = int(w.shape[0]), int(w.shape[1])
    M = x.numel() // K if K else 0
    y = out if out is not None else torch.empty(tuple(x.shape[:-1]) + (N,), dtype=out_dtype, device=x.device)
    code = CSA_F32 if out_dtype == torch.float32 else CSA_BF16
    _check(load_library().csa_project(_ptr(x), _ptr(w), int(M), N, K, code, _ptr(y), _stream_handle()))
    return y


def query_projection(c, wq, H=64):
    """Indexer queries q [B, S, H, D] (bf16, head-major) from the low-rank
    latents c [B, S, r] and W_q [H*D, r]."""
    if c.dim() != 3 or wq.dim() != 2 or wq.shape[0] % H:
        raise ValueError(f"expected c [B, S, r] and W_q [H*D, r] with H={H}: c {tuple(c.shape)} W_q {tuple(wq.shape)}")
    B, S = c.shape[0], c.shape[1]
    return project(c, wq).view(B, S, H, wq.shape[0] // H)


def head_weight_projection(x, ww):
    """Indexer head weights w [B, S, H] (fp32) from hidden states x [B, S, d]
    and W_w [H, d]."""
    if x.dim() != 3 or ww.dim() != 2:
        raise ValueError(f"expected x [B, S, d] and W_w [H, d]: x {tuple(x.shape)} W_w {tuple(ww.shape)}")
    return project(x, ww, out_dtype=_torch().float32)


def compress_keys(z, wk, m=4):
    """Compressed keys k [B, S/m, D] (bf16): key s is W_k [D, m*d_z] applied to
    the m token vectors z[b, m*s .. m*s+m-1] side by side (z [B, S, d_z])."""
    if z.dim() != 3 or wk.dim() != 2:
        raise ValueError(f"expected z [B, S, d_z] and W_k [D, m*d_z]: z {tuple(z.shape)} W_k {tuple(wk.shape)}")
    B, S, dz = z.shape
    if S % m:
        raise ValueError("S must be a multiple of m")
    if not z.is_contiguous():
        raise ValueError("z must be contiguous")
    return project(z.view(B, S // m, m * dz), wk)
