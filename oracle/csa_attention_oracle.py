"""CPU oracle for CSA stage 4: sparse attention over the selected keys.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
``bench.py``'s ``cpu_baseline`` leg may import or run this module.  It shares
no code with the HIP library.

What it computes.  Once the lightning indexer has picked a query's top-k
compressed keys, the attention step of Compressed Sparse Attention touches
only those keys (StreamIndex paper, abstract; the Multi-layer Indexer blog
post describes each DeepSeek Sparse Attention layer attending to the 2048
entries its indexer picks).  The pages give no formula for that step; the
reading here is
standard scaled softmax attention restricted to the selected entries, with
every query head attending to the same selected compressed key and value rows
(one shared compressed entry per key position, as the indexer shares one
compressed key across its heads):

    o[b, t, h, :] = sum_{e valid}  p_e * v[b, idx[b, t, e], :]
    p_e = exp(z_e - max z) / sum_e' exp(z_e' - max z)
    z_e = scale * q[b, t, h, :] . k[b, idx[b, t, e], :]

An entry is valid when 0 <= idx < T; entries are taken as listed (an index
listed twice counts twice).  A row with no valid entry gives o = 0.

Everything is float64 on exactly widened bf16 inputs, one query row at a
time.
"""
from __future__ import annotations

import numpy as np

from .csa_oracle import decode_bf16


def attention_row(q_row: np.ndarray, k_sel: np.ndarray, v_sel: np.ndarray, scale: float) -> np.ndarray:
    """Softmax attention of the H query heads q_row [H, Dk] over the selected
    key rows k_sel [n, Dk] and value rows v_sel [n, Dv] -> [H, Dv] (float64)."""
    H = q_row.shape[0]
    if k_sel.shape[0] == 0:
        return np.zeros((H, v_sel.shape[1]), dtype=np.float64)
    z = scale * (q_row @ k_sel.T)                      # [H, n]
    z = z - z.max(axis=1, keepdims=True)
    e = np.exp(z)
    p = e / e.sum(axis=1, keepdims=True)
    return p @ v_sel


def oracle_attention(prob, idx: np.ndarray, scale: float, rows=None) -> np.ndarray:
    """o [B, S_q, H, Dv] (float64) for the attention problem `prob` (dict with
    bf16 bit arrays q [B,S_q,H,Dk], k [B,T,Dk], v [B,T,Dv]) and selections
    idx [B, S_q, n_sel] int32.  rows: optional list of query rows to compute
    (others left 0)."""
    q = prob["q"]
    B, S_q, H, _ = q.shape
    T = prob["k"].shape[1]
    Dv = prob["v"].shape[2]
    out = np.zeros((B, S_q, H, Dv), dtype=np.float64)
    rr = range(S_q) if rows is None else rows
    for b in range(B):
        kb = decode_bf16(prob["k"][b])
        vb = decode_bf16(prob["v"][b])
        for t in rr:
            sel = np.asarray(idx[b, t], dtype=np.int64)
            sel = sel[(sel >= 0) & (sel < T)]
            out[b, t] = attention_row(decode_bf16(q[b, t]), kb[sel], vb[sel], scale)
    return out
