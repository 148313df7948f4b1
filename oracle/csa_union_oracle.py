"""CPU oracle for the multi-layer union of selections.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
``bench.py``'s ``cpu_baseline`` leg may import or run this module.  It shares
no code with the HIP library.

What it computes.  The FlashMemory-DeepSeek-V4 review ("What carries the
argument") places the Memory Indexer on three layers (10, 12 and 20) and
combines their keep decisions with a logical OR while decoding; its free
parameters list a decode trigger interval of tau = 64 steps between
selections.  Read as: per query row, the selected set is the union of the
layers' selected index sets (each layer's own threshold selection), kept
between refreshes.  The union is reported in ascending index order with its
true size; a cap keeps the smallest indices.
"""
from __future__ import annotations

import numpy as np

from .csa_oracle import oracle_threshold


def oracle_union(lists, T: int, cap: int):
    """lists: sequence of int arrays [..., width_i] with equal leading shapes.
    Returns (idx [..., cap] int32 ascending then -1, count [...] int32)."""
    lead = np.asarray(lists[0]).shape[:-1]
    out = np.full(lead + (cap,), -1, dtype=np.int32)
    cnt = np.zeros(lead, dtype=np.int32)
    for pos in np.ndindex(*lead):
        s = set()
        for li in lists:
            for v in np.asarray(li)[pos].tolist():
                if 0 <= v < T:
                    s.add(int(v))
        u = sorted(s)
        cnt[pos] = len(u)
        out[pos][: min(cap, len(u))] = u[:cap]
    return out, cnt


def oracle_multilayer(probs, prob_threshold: float, cap: int, union_cap: int, logit_bias: float = 0.0):
    """Union over layers of each layer's threshold selection (top-`cap` of its
    survivors), for problems `probs` that share B, S_q and T."""
    sels = [oracle_threshold(p, prob_threshold, logit_bias, cap=cap)[0] for p in probs]
    return oracle_union(sels, probs[0]["T"], union_cap)
