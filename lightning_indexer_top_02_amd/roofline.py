"""Algorithmic work counts and MI355X roofline denominators.

Counts only what the method must do:
* prefill: 2*H*D flops per (query, visible key) pair, over rows that have more
  visible keys than k (a row with vis <= k selects every visible key and needs
  no score); the all-visible count is reported beside it;
* decode: bytes of K, Q, w and the output indices, each moved once;
* sparse attention: bytes of the selected key and value rows, Q, the index
  rows and the output, each moved once.
"""
from __future__ import annotations

# MI355X vendor peaks (dense): bf16 MFMA 2.5 PFLOP/s, HBM3E 8 TB/s.
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBPS = 8000.0
NUM_CUS = 256
CLOCK_GHZ = 2.4


def row_visible(t_abs: int, m: int, T: int, causal: bool = True, kv_len=None) -> int:
    v = t_abs // m + 1 if causal else T
    v = min(v, T)
    if kv_len is not None:
        v = min(v, max(int(kv_len), 0))
    return max(v, 0)


def visible_pairs(S_q: int, q_pos0: int, m: int, T: int, topk: int, causal: bool = True, B: int = 1):
    """(needed pairs, all visible pairs) summed over B*S_q rows, closed form per row range."""
    need = allv = 0
    for i in range(S_q):
        v = row_visible(q_pos0 + i, m, T, causal)
        allv += v
        if v > topk:
            need += v
    return need * B, allv * B


def prefill_flops(H: int, D: int, pairs: int) -> int:
    return 2 * H * D * pairs


def decode_bytes(B: int, S_q: int, T: int, H: int, D: int, topk: int, elem: int = 2) -> int:
    return B * T * D * elem + B * S_q * H * D * elem + B * S_q * H * 4 + B * S_q * topk * 4


def attention_bytes(rows: int, n_valid: int, H: int, Dk: int, Dv: int, n_sel: int, elem: int = 2) -> int:
    """Sparse attention: the selected key and value rows (n_valid entries over
    all rows), the queries, the index rows and the fp32 output, each moved once."""
    return n_valid * (Dk + Dv) * elem + rows * H * Dk * elem + rows * n_sel * 4 + rows * H * Dv * 4


def materialised_score_bytes(B: int, S: int, H: int, T: int) -> int:
    """Size of the fp32 [B, S, H_I, T] score tensor the streaming method avoids."""
    return B * S * H * T * 4


def interleaved_pairs(S_q: int, q_pos0: int, m: int, T: int, P: int, k_local: int, causal: bool = True,
                      B: int = 1) -> int:
    """Needed (query, key) pairs of the interleaved variant: partition p of a
    row holds its visible keys s = p, p+P, ...; a partition with at most
    k_local of them keeps them all and needs no score."""
    need = 0
    for i in range(S_q):
        v = row_visible(q_pos0 + i, m, T, causal)
        for p in range(P):
            n = (v - p + P - 1) // P if v > p else 0
            if n > k_local:
                need += n
    return need * B
