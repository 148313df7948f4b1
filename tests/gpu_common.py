"""Helpers for the GPU parity tests: move seeded inputs to the device and
compare the HIP library's selections with the CPU oracle.

Tolerance rule for bf16 inputs (fp32 accumulation on the GPU vs fp64 in the
oracle): with rms = RMS of the row's visible oracle scores and
floor = rms / 256,
  * every returned score s: |I_gpu - I_ref| <= 2e-3 * max(|I_ref|, floor);
  * an index may be in only one of the two sets only if its oracle score is
    within 2e-3 * max(|v_n|, floor) of the oracle's n-th largest score v_n.
Integer-valued inputs must match exactly (sets, and scores bitwise).
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch
from threadpoolctl import threadpool_limits

import oracle

REL = 2e-3
FLOOR_DIV = 256.0


def to_device(prob, device="cuda"):
    if prob["dtype"] == "bf16":
        q = torch.from_numpy(np.ascontiguousarray(prob["q"]).view(np.int16)).view(torch.bfloat16)
        k = torch.from_numpy(np.ascontiguousarray(prob["k"]).view(np.int16)).view(torch.bfloat16)
    else:
        q = torch.from_numpy(np.ascontiguousarray(prob["q"], dtype=np.float32))
        k = torch.from_numpy(np.ascontiguousarray(prob["k"], dtype=np.float32))
    w = torch.from_numpy(np.ascontiguousarray(prob["w"], dtype=np.float32))
    kv = None
    if prob.get("kv_len") is not None:
        kv = torch.from_numpy(np.asarray(prob["kv_len"], dtype=np.int32)).to(device)
    return q.to(device), k.to(device), w.to(device), kv


def valid_prefix_ok(row, n):
    """First n entries valid and distinct, the rest -1."""
    head = row[:n]
    return (head >= 0).all() and len(set(head.tolist())) == n and (row[n:] == -1).all()


def check_exact(gpu_idx, ref_idx, gpu_score=None, ref_score=None):
    """Integer inputs: identical sets per row (and identical scores per index)."""
    g = np.asarray(gpu_idx)
    r = np.asarray(ref_idx)
    assert g.shape == r.shape
    G = g.reshape(-1, g.shape[-1])
    Rr = r.reshape(-1, r.shape[-1])
    bad = [i for i in range(G.shape[0]) if sorted(G[i].tolist()) != sorted(Rr[i].tolist())]
    assert not bad, f"{len(bad)} rows differ, first {bad[:5]}: gpu {sorted(G[bad[0]].tolist())[:12]} ref {sorted(Rr[bad[0]].tolist())[:12]}"
    if gpu_score is not None:
        GS = np.asarray(gpu_score).reshape(G.shape)
        RS = np.asarray(ref_score).reshape(G.shape)
        for i in range(G.shape[0]):
            gm = dict(zip(G[i].tolist(), GS[i].tolist()))
            rm = dict(zip(Rr[i].tolist(), RS[i].tolist()))
            assert gm == rm, f"row {i} scores differ"


def _pool_size():
    return max(1, min(16, os.cpu_count() or 1))


def map_rows(fn, items, say=None, chunk=512):
    """fn over items in a thread pool (numpy releases the GIL in its matmuls
    and ufuncs), BLAS held to one thread per worker; results in item order.
    An AssertionError in any item propagates.  `say` gets a progress line
    after every `chunk` items."""
    items = list(items)
    if len(items) <= 4:
        return [fn(x) for x in items]
    out = []
    with threadpool_limits(1):
        with ThreadPoolExecutor(_pool_size()) as ex:
            for c0 in range(0, len(items), chunk):
                out.extend(ex.map(fn, items[c0:c0 + chunk]))
                if say is not None:
                    say(f"  checked {len(out)} of {len(items)} rows")
    return out


def check_tolerance(prob, rows, gpu_idx, gpu_score, topk, b_list=None, say=None):
    """bf16 inputs: the tolerance rule above, row by row (rows = query rows of
    gpu_idx[b, r]); rows are checked in parallel threads."""
    scorer = oracle.RowScorer(prob)
    B = prob["B"]

    def one(br):
        b, r, i = br
        I = scorer(b, i)
        vis = I.shape[0]
        n = min(topk, vis)
        g = np.asarray(gpu_idx[b, r])
        assert valid_prefix_ok(g, n), f"row {i}: bad padding/duplicates"
        gs = g[:n]
        assert (gs < vis).all(), f"row {i}: index beyond visible range"
        if vis == 0:
            return 0, 0.0, 0
        floor = float(np.sqrt(np.mean(I * I))) / FLOOR_DIV
        ref = oracle.select_topk(I, n)
        vn = I[ref].min() if n > 0 else 0.0
        band = REL * max(abs(vn), floor)
        diff = set(gs.tolist()) ^ set(ref.tolist())
        for s in diff:
            assert abs(I[s] - vn) <= band, f"row {i}: index {s} score {I[s]} outside band around v_n={vn}"
        mrel = 0.0
        if gpu_score is not None:
            sc = np.asarray(gpu_score[b, r][:n], dtype=np.float64)
            err = np.abs(sc - I[gs])
            lim = REL * np.maximum(np.abs(I[gs]), floor)
            assert (err <= lim).all(), f"row {i}: score error {err.max()} beyond tolerance"
            mrel = float((err / np.maximum(np.abs(I[gs]), floor)).max()) if n else 0.0
        return len(diff) // 2, mrel, 1

    items = [(b, r, int(i)) for b in (range(B) if b_list is None else b_list) for r, i in enumerate(rows)]
    res = map_rows(one, items, say)
    return dict(rows=sum(x[2] for x in res), swaps=sum(x[0] for x in res),
                max_rel=max([x[1] for x in res], default=0.0))
