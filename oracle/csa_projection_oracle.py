"""CPU oracle for the producers of the indexer's inputs (query, head weights,
compressed keys).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
``bench.py``'s ``cpu_baseline`` leg may import or run this module.  It shares
no code with the HIP library.

What it computes.  The pages name the pieces but give no formulas: the
FlashMemory review lists a low-rank query projection of dimension r = 2048
(q_lora_rank) in the Memory Indexer's query encoder, and StreamIndex (abstract)
scores keys compressed by a ratio m (T = S/m, m = 4 for V4-Flash).  The
readings here are the plainest linear ones:

    q[b, t, j, :] = (W_q c[b, t])[j*D : (j+1)*D]        c[b, t] in R^r
    w[b, t, j]    = (W_w x[b, t])[j]                    x[b, t] in R^d
    k[b, s, :]    = W_k concat(z[b, m*s], ..., z[b, m*s + m - 1])

with W_q [H*D, r], W_w [H, d], W_k [D, m*d_z] and row-major outputs (head j's
D values contiguous).  All three are one operation, y = X W^T over bf16
operands; here it is float64 on exactly widened bf16 values.
"""
from __future__ import annotations

import numpy as np

from .csa_oracle import decode_bf16


def project(x_bits: np.ndarray, w_bits: np.ndarray) -> np.ndarray:
    """y [..., N] = x [..., K] . w [N, K]^T, float64 (bf16 bit-pattern inputs)."""
    x = decode_bf16(x_bits)
    w = decode_bf16(w_bits)
    return x @ w.T


def project_abs(x_bits: np.ndarray, w_bits: np.ndarray) -> np.ndarray:
    """sum_k |x_k| |w_nk|, the scale of the rounding error of each output."""
    return np.abs(decode_bf16(x_bits)) @ np.abs(decode_bf16(w_bits)).T


def oracle_query(c_bits: np.ndarray, wq_bits: np.ndarray, H: int, D: int) -> np.ndarray:
    """q [B, S, H, D] from the low-rank latents c [B, S, r] and W_q [H*D, r]."""
    B, S, _ = c_bits.shape
    return project(c_bits, wq_bits).reshape(B, S, H, D)


def oracle_head_weights(x_bits: np.ndarray, ww_bits: np.ndarray) -> np.ndarray:
    """w [B, S, H] from the hidden states x [B, S, d] and W_w [H, d]."""
    return project(x_bits, ww_bits)


def oracle_compress_keys(z_bits: np.ndarray, wk_bits: np.ndarray, m: int) -> np.ndarray:
    """k [B, S/m, D]: compressed key s is W_k applied to the concatenation of
    the m token vectors m*s .. m*s + m - 1 (z [B, S, d_z], W_k [D, m*d_z])."""
    B, S, dz = z_bits.shape
    if S % m:
        raise ValueError("S must be a multiple of m")
    groups = z_bits.reshape(B, S // m, m * dz)          # token m*s+i fills columns i*d_z .. (i+1)*d_z - 1
    return project(groups, wk_bits)
