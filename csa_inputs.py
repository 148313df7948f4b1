"""Seeded synthetic inputs for the CSA lightning-indexer top-k path.

This module only draws random numbers and lays them out; it holds none of
the indexer's arithmetic (no scores, no selection).  Both the CPU oracle
(``oracle/``) and the HIP path (tests, ``bench.py``) take their inputs from
here, so the two see bit-identical data.

Workload shapes follow the V4-Flash indexer dimensions the StreamIndex paper
(arXiv 2605.02568, abstract) measures on: H_I = 64 indexer heads over
keys compressed by m = 4.  The paper says only that its inputs are synthetic
and shaped like V4's indexer step, with no value distribution, so the recipe
here is:

* bf16 configs: q, k ~ N(0,1)/sqrt(d_I) drawn in fp32 and rounded to bf16
  with round-to-nearest-even; w ~ N(0,1)/sqrt(H_I) kept in fp32.
* the tiny exact config: q, k integers uniform in [-4, 4] stored as fp32,
  w integers uniform in [-2, 2] -- every score is an exact small integer,
  which floods the selection with ties.
* decode: 64 planted keys per sequence, each 4 x the unit "query
  direction" u = normalise(sum_j max(w_j, 0) * q_j), at positions drawn
  without replacement.

A config is a plain dict; arrays are numpy (bf16 data as uint16 bit patterns).
"""
from __future__ import annotations

import numpy as np

BF16 = "bf16"
F32 = "f32"


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round-to-nearest-even); return uint16 bits.

    Inputs are finite by construction (no NaN handling needed)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def _problem(dtype, B, S_q, T, H, D, m, q_pos0, topk, q, k, w, kv_len=None,
             name="", seed=None, causal=True):
    return dict(dtype=dtype, B=B, S_q=S_q, T=T, H=H, D=D, m=m, q_pos0=q_pos0,
                topk=topk, q=q, k=k, w=w, kv_len=kv_len, name=name, seed=seed,
                causal=causal)


def make_integer(B=1, S_q=1024, T=256, H=4, D=32, m=4, topk=64, q_pos0=0,
                 seed=1001, qk_range=4, w_range=2, name="tiny-exact"):
    """Integer-valued fp32 problem (exact scores, heavy ties)."""
    rng = np.random.default_rng(seed)
    q = rng.integers(-qk_range, qk_range + 1, size=(B, S_q, H, D)).astype(np.float32)
    k = rng.integers(-qk_range, qk_range + 1, size=(B, T, D)).astype(np.float32)
    w = rng.integers(-w_range, w_range + 1, size=(B, S_q, H)).astype(np.float32)
    return _problem(F32, B, S_q, T, H, D, m, q_pos0, topk, q, k, w, name=name, seed=seed)


def make_gaussian_bf16(B, S_q, T, H, D, m, topk, q_pos0=0, seed=0, name=""):
    """q, k ~ N(0,1)/sqrt(D) rounded to bf16; w ~ N(0,1)/sqrt(H) fp32."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, S_q, H, D), dtype=np.float32)
    q *= np.float32(1.0 / np.sqrt(D))
    qb = f32_to_bf16_bits(q)
    del q
    k = rng.standard_normal((B, T, D), dtype=np.float32)
    k *= np.float32(1.0 / np.sqrt(D))
    kb = f32_to_bf16_bits(k)
    del k
    w = rng.standard_normal((B, S_q, H), dtype=np.float32)
    w *= np.float32(1.0 / np.sqrt(H))
    return _problem(BF16, B, S_q, T, H, D, m, q_pos0, topk, qb, kb, w, name=name, seed=seed)


def make_decode(B=32, context=131072, m=4, H=64, D=128, topk=2048, n_planted=64,
                S_q=1, seed=1004, name="decode-scan"):
    """Decode: B sequences, S_q queries each at the end of a `context`-token
    sequence, T = context/m compressed keys, with planted high-score keys."""
    T = context // m
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, S_q, H, D), dtype=np.float32) * np.float32(1.0 / np.sqrt(D))
    k = rng.standard_normal((B, T, D), dtype=np.float32) * np.float32(1.0 / np.sqrt(D))
    w = rng.standard_normal((B, S_q, H), dtype=np.float32) * np.float32(1.0 / np.sqrt(H))
    planted = np.zeros((B, n_planted), dtype=np.int64)
    for b in range(B):
        pos = np.sort(rng.choice(T, size=n_planted, replace=False))
        # query direction of the sequence's first query: positive-weighted head mix
        u = (np.maximum(w[b, 0], 0.0)[:, None].astype(np.float64) * q[b, 0].astype(np.float64)).sum(0)
        nrm = np.linalg.norm(u)
        u = u / nrm if nrm > 0 else np.ones(D) / np.sqrt(D)
        k[b, pos, :] = (4.0 * u).astype(np.float32)[None, :]
        planted[b] = pos
    q_pos0 = context - S_q
    prob = _problem(BF16, B, S_q, T, H, D, m, q_pos0, topk, f32_to_bf16_bits(q),
                    f32_to_bf16_bits(k), w, name=name, seed=seed)
    prob["planted"] = planted
    return prob


def make_attention(B, S_q, T, H=64, Dk=128, Dv=128, n_sel=2048, seed=0, pad=0, name=""):
    """Inputs of the sparse attention step: q [B,S_q,H,Dk], k [B,T,Dk] and
    v [B,T,Dv] ~ N(0,1) rounded to bf16, and per query row n_sel distinct key
    indices drawn uniformly from [0, T) with the last `pad` entries set to -1."""
    rng = np.random.default_rng(seed)
    q = f32_to_bf16_bits(rng.standard_normal((B, S_q, H, Dk), dtype=np.float32))
    k = f32_to_bf16_bits(rng.standard_normal((B, T, Dk), dtype=np.float32))
    v = f32_to_bf16_bits(rng.standard_normal((B, T, Dv), dtype=np.float32))
    idx = np.empty((B, S_q, n_sel), dtype=np.int32)
    for b in range(B):
        for t in range(S_q):
            idx[b, t] = rng.choice(T, size=n_sel, replace=False)
    if pad:
        idx[:, :, n_sel - pad:] = -1
    return dict(B=B, S_q=S_q, T=T, H=H, Dk=Dk, Dv=Dv, n_sel=n_sel, q=q, k=k, v=v, idx=idx,
                scale=float(1.0 / np.sqrt(Dk)), seed=seed, name=name)


# --- the five named workloads -------------------------------------------------

def config(n: int):
    """Return synthetic problem #n (1..5); seed = 1000 + n."""
    if n == 1:
        return make_integer(seed=1001, name="tiny-exact S=1024 T=256 H=4 D=32 k=64")
    if n == 2:
        return make_gaussian_bf16(1, 16384, 4096, 64, 128, 4, 2048, q_pos0=0, seed=1002,
                                  name="V4-Flash prefill S=16384 T=4096 H=64 D=128 k=2048")
    if n == 3:
        return make_gaussian_bf16(1, 65536, 16384, 64, 128, 4, 2048, q_pos0=0, seed=1003,
                                  name="long prefill S=65536 T=16384 H=64 D=128 k=2048")
    if n == 4:
        return make_decode(seed=1004, name="decode B=32 ctx=131072 T=32768 H=64 D=128 k=2048")
    if n == 5:
        S_total = 1 << 20
        S_q = 8192
        return make_gaussian_bf16(1, S_q, S_total // 4, 64, 128, 4, 2048, q_pos0=S_total - S_q,
                                  seed=1005,
                                  name="million-token tail S_q=8192 q_pos0=1040384 T=262144 k=2048")
    raise ValueError(f"no config {n}")


def scaled_config2(S_q=2048, T=None, seed=1002):
    """Config-2 distributions at a smaller size (T = S_q/4 keeps the causal shape)."""
    if T is None:
        T = S_q // 4
    return make_gaussian_bf16(1, S_q, T, 64, 128, 4, 2048, q_pos0=0, seed=seed,
                              name=f"V4-Flash prefill scaled S={S_q} T={T}")


def sample_rows(S_q: int, n: int, seed: int, must=()):
    """A fixed seeded sample of query rows (sorted, unique), always containing `must`."""
    rng = np.random.default_rng(seed)
    n = min(n, S_q)
    rows = set(int(r) for r in must if 0 <= r < S_q)
    extra = rng.choice(S_q, size=n, replace=False)
    for r in extra:
        if len(rows) >= n:
            break
        rows.add(int(r))
    return np.array(sorted(rows), dtype=np.int64)


def make_projection(M, N, K, seed=0, kind="gauss"):
    """Operands of a projection y = x . w^T as bf16 bit patterns: x [M, K] and
    w [N, K].  kind "gauss": x ~ N(0,1), w ~ N(0,1)/sqrt(K) (unit-scale
    outputs), rounded to bf16; kind "int": integers uniform in {-1, 0, 1}
    (every sum exact, every output a bf16-representable integer for K <= 256)."""
    rng = np.random.default_rng(seed)
    if kind == "int":
        x = rng.integers(-1, 2, size=(M, K)).astype(np.float32)
        w = rng.integers(-1, 2, size=(N, K)).astype(np.float32)
    else:
        x = rng.standard_normal((M, K), dtype=np.float32)
        w = rng.standard_normal((N, K), dtype=np.float32) * np.float32(1.0 / np.sqrt(K))
    return f32_to_bf16_bits(x), f32_to_bf16_bits(w)
