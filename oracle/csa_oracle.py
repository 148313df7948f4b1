"""CPU oracle for the CSA lightning-indexer top-k step.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
``bench.py``'s ``cpu_baseline`` leg may import or run this module.  The HIP
library never calls it and shares no code with it; the product path fails
loudly when the HIP library is missing instead of falling back here.

What it computes (sources: the StreamIndex paper, arXiv 2605.02568,
abstract; the FlashMemory-DeepSeek-V4 machine review, "What carries the
argument" and the axiom ledger; DeepSeek Sparse Attention as described in
the Multi-layer Indexer blog post):

* DeepSeek-V3.2/V4 Compressed Sparse Attention scores compressed keys with a
  "lightning indexer" and keeps the top-k keys per query (StreamIndex
  abstract).  The score is a dot product of the query with each compressed key,
  taken per indexer head, passed through ReLU and fused across heads
  (FlashMemory review, axiom ledger, Eq. 4 as cited there; "native Lightning
  Indexer" uses ReLU, "What carries the argument"):

      I[t, s] = sum_j  w[t, j] * max(q[t, j] . k[s], 0)

  over H_I heads j, with no extra scale or bias (a positive scale is the
  caller's to fold into w).
* Keys are compressed by ratio m (V4-Flash: m = 4, StreamIndex abstract).
  Causality on compressed keys is read as: the query at absolute position t
  sees keys s <= floor(t / m).
* Selection is an exact top-k with ties broken toward the lower key index;
  the materialise-then-top-k path is the ground truth the streaming method
  must match (StreamIndex abstract: set-overlap recall is bit-exact at small S).
* Threshold variant: rather than a top-k of fixed size, FlashMemory's Memory
  Indexer keeps each key whose sigmoid-mapped score lies above 0.5 ("What
  carries the argument"; free parameter "classification threshold").
  Read as sigma(I + bias) > tau, i.e. I > logit(tau) - bias, strict.
* Interleaved variant: Interleaved DeepSeek Sparse Attention places tokens
  in an interleaved layout across devices; each device selects locally and
  the union of local selections is meant to cover the global top tokens
  (Machine Press story, summary).  Read as: partition p holds keys with
  s mod P == p and keeps its own top-k_local; recall = |union ∩ G| / |G|.

Everything is float64 on exactly widened inputs (bf16 bit patterns shifted
into fp32, then widened).  The scores are computed one query row at a time
with a BLAS matmul; no [B, S, H_I, T] tensor is built.
"""
from __future__ import annotations

import itertools
import math

import numpy as np

# ---------------------------------------------------------------------------
# input widening


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float64 values.

    A bf16 value is the upper half of an IEEE binary32 word, so shifting its
    bits left by 16 gives the fp32 word exactly."""
    b = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def widen(arr: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return decode_bf16(arr)
    if dtype == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# visibility


def visible_count(t_abs: int, m: int, T: int, causal: bool = True, kv_len=None) -> int:
    """Number of keys query position t_abs may score: keys 0..vis-1.

    Causal: s <= floor(t_abs / m).  Then capped by T and by kv_len (if given)."""
    vis = (t_abs // m) + 1 if causal else T
    vis = min(vis, T)
    if kv_len is not None:
        vis = min(vis, max(int(kv_len), 0))
    return max(vis, 0)


def _row_vis(prob, b, i):
    kv = None if prob.get("kv_len") is None else prob["kv_len"][b]
    return visible_count(prob["q_pos0"] + i, prob["m"], prob["T"], prob.get("causal", True), kv)


# ---------------------------------------------------------------------------
# scores


def row_scores(q_row: np.ndarray, k_vis: np.ndarray, w_row: np.ndarray) -> np.ndarray:
    """I[s] = sum_j w[j] * max(q[j] . k[s], 0) for the given visible keys.

    q_row [H, D], k_vis [vis, D], w_row [H], all float64.  Returns [vis]
    float64 with -0.0 turned into +0.0."""
    logits = q_row @ k_vis.T                      # [H, vis]: per-head dot products
    relu = np.maximum(logits, 0.0)
    score = (w_row[:, None] * relu).sum(axis=0)   # head-weighted fusion
    return score + 0.0                            # -0.0 + 0.0 == +0.0


class _Widened:
    """Per-problem cache of float64 keys (queries are widened row by row)."""

    def __init__(self, prob):
        self.prob = prob
        self.k = [widen(prob["k"][b], prob["dtype"]) for b in range(prob["B"])]

    def q_row(self, b, i):
        return widen(self.prob["q"][b, i], self.prob["dtype"])

    def w_row(self, b, i):
        return np.asarray(self.prob["w"][b, i], dtype=np.float32).astype(np.float64)

    def scores(self, b, i):
        vis = _row_vis(self.prob, b, i)
        if vis == 0:
            return np.zeros(0)
        return row_scores(self.q_row(b, i), self.k[b][:vis], self.w_row(b, i))


def row_score_vector(prob, b, i):
    """Float64 scores of query row i of sequence b against its visible keys."""
    return _Widened(prob).scores(b, int(i))


class RowScorer:
    """Scores many rows of one problem, widening the keys once."""

    def __init__(self, prob):
        self._w = _Widened(prob)

    def __call__(self, b, i):
        return self._w.scores(b, int(i))


# ---------------------------------------------------------------------------
# selection


def order_desc(I: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Sort the key indices `idx` by (score descending, index ascending)."""
    idx = np.asarray(idx, dtype=np.int64)
    return idx[np.lexsort((idx, -I[idx]))]


def select_topk(I: np.ndarray, n: int) -> np.ndarray:
    """Exact top-n of I with ties at the cut going to the lower index.

    v = the n-th largest score; keep every index scoring above v, then the
    lowest-index ones among those equal to v until n are kept.  Returned in
    (score desc, index asc) order."""
    vis = I.shape[0]
    n = min(n, vis)
    if n <= 0:
        return np.zeros(0, dtype=np.int64)
    v = np.partition(I, vis - n)[vis - n]
    above = np.nonzero(I > v)[0]
    equal = np.nonzero(I == v)[0]            # ascending index order
    sel = np.concatenate([above, equal[: n - above.shape[0]]])
    return order_desc(I, sel)


def _rows_arg(prob, rows):
    return np.arange(prob["S_q"]) if rows is None else np.asarray(rows, dtype=np.int64)


def oracle_topk(prob, topk=None, rows=None):
    """Top-k indices and scores for every (b, row).

    Returns (idx [B, R, topk] int32 padded with -1, score [B, R, topk] fp32
    padded with -inf, vis [B, R] int64); R = len(rows) or S_q.  Each row's
    indices are in (score desc, index asc) order."""
    topk = prob["topk"] if topk is None else topk
    rows = _rows_arg(prob, rows)
    B = prob["B"]
    out_i = np.full((B, len(rows), topk), -1, dtype=np.int32)
    out_s = np.full((B, len(rows), topk), -np.inf, dtype=np.float32)
    vis_out = np.zeros((B, len(rows)), dtype=np.int64)
    wd = _Widened(prob)
    for b in range(B):
        for r, i in enumerate(rows):
            I = wd.scores(b, int(i))
            vis_out[b, r] = I.shape[0]
            sel = select_topk(I, topk)
            out_i[b, r, : sel.shape[0]] = sel
            out_s[b, r, : sel.shape[0]] = I[sel].astype(np.float32)
    return out_i, out_s, vis_out


def logit_threshold(prob_threshold: float, logit_bias: float) -> float:
    """theta with sigma(I + bias) > tau  <=>  I > theta (host double)."""
    t = float(np.float32(prob_threshold))
    b = float(np.float32(logit_bias))
    return math.log(t / (1.0 - t)) - b


def oracle_threshold(prob, prob_threshold=0.5, logit_bias=0.0, cap=None, rows=None):
    """Keys with I > logit(tau) - bias; count is the true survivor count and
    idx holds the first min(cap, count) survivors in (score desc, index asc)
    order, padded with -1 (scores padded with -inf)."""
    cap = prob["topk"] if cap is None else cap
    theta = logit_threshold(prob_threshold, logit_bias)
    rows = _rows_arg(prob, rows)
    B = prob["B"]
    out_i = np.full((B, len(rows), cap), -1, dtype=np.int32)
    out_s = np.full((B, len(rows), cap), -np.inf, dtype=np.float32)
    count = np.zeros((B, len(rows)), dtype=np.int32)
    wd = _Widened(prob)
    for b in range(B):
        for r, i in enumerate(rows):
            I = wd.scores(b, int(i))
            surv = order_desc(I, np.nonzero(I > theta)[0])
            count[b, r] = surv.shape[0]
            keep = surv[:cap]
            out_i[b, r, : keep.shape[0]] = keep
            out_s[b, r, : keep.shape[0]] = I[keep].astype(np.float32)
    return out_i, count, out_s


def oracle_interleaved(prob, P, k_local, rows=None):
    """Partition p = keys with s mod P == p; each keeps its own top-k_local
    (same total order).  idx [B, R, P*k_local]: partition p's list starts at
    p*k_local, (score desc, index asc), padded with -1."""
    rows = _rows_arg(prob, rows)
    B = prob["B"]
    out_i = np.full((B, len(rows), P * k_local), -1, dtype=np.int32)
    out_s = np.full((B, len(rows), P * k_local), -np.inf, dtype=np.float32)
    wd = _Widened(prob)
    for b in range(B):
        for r, i in enumerate(rows):
            I = wd.scores(b, int(i))
            vis = I.shape[0]
            for p in range(P):
                part = np.arange(p, vis, P, dtype=np.int64)
                if part.shape[0] == 0:
                    continue
                local = select_topk(I[part], k_local)     # positions within the partition
                sel = part[local]
                out_i[b, r, p * k_local: p * k_local + sel.shape[0]] = sel
                out_s[b, r, p * k_local: p * k_local + sel.shape[0]] = I[sel].astype(np.float32)
    return out_i, out_s


def oracle_recall(sel: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per row |set(sel) ∩ set(ref)| / |set(ref)|, ignoring -1 entries.
    An empty reference set has recall 1."""
    sel = np.asarray(sel).reshape(-1, np.asarray(sel).shape[-1])
    ref = np.asarray(ref).reshape(-1, np.asarray(ref).shape[-1])
    out = np.zeros(sel.shape[0], dtype=np.float64)
    for r in range(sel.shape[0]):
        g = set(int(x) for x in ref[r] if x >= 0)
        u = set(int(x) for x in sel[r] if x >= 0)
        out[r] = 1.0 if not g else len(g & u) / len(g)
    return out


# ---------------------------------------------------------------------------
# exhaustive enumeration (tiny integer inputs only)


def exact_int_scores(q_row, k_rows, w_row):
    """Scores with Python integers (inputs must be integer-valued)."""
    out = []
    for kr in k_rows:
        tot = 0
        for qj, wj in zip(q_row, w_row):
            dot = 0
            for a, c in zip(qj, kr):
                dot += int(a) * int(c)
            tot += int(wj) * max(dot, 0)
        out.append(tot)
    return out


def exhaustive_topk(scores, n):
    """Among all size-n subsets of range(len(scores)), the one with the largest
    exact score sum; among equal sums, the lexicographically smallest sorted
    tuple.  Pure Python, O(C(len, n))."""
    n = min(n, len(scores))
    best, best_sum = None, None
    for comb in itertools.combinations(range(len(scores)), n):   # lexicographic order
        s = sum(scores[i] for i in comb)
        if best_sum is None or s > best_sum:
            best, best_sum = comb, s
    return tuple(best) if best is not None else tuple()
