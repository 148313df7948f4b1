#!/usr/bin/env python3
"""Throughput of the CSA lightning-indexer top-k on one MI355X.

A step is one csa_index_topk_prefill call over the V4-Flash-shaped prefill
workload (B=1, S=16384 queries, m=4 so T=4096 compressed keys, H_I=64,
d_I=128, top-k=2048; bf16 q/k ~ N(0,1)/sqrt(128), fp32 w ~ N(0,1)/8; causal)
with inputs resident in HBM.  value = algorithmic prefill TFLOP/s: 2*H*D flops
per (query, visible key) pair over rows with more visible keys than k.

Also reported on the same JSON line:
  roofline      the prefill kernel against the bf16 MFMA peak (HIP-event time
                of each launch on the library's stream, in a pass of its own
                after the timed region);
  decode        the decode scan (B=32 x T=32768, k=2048) in GB/s against HBM
                peak, K rotated over 4 copies so the 256 MB MALL cannot hold it;
  attention     sparse attention over 2048 selected of T=32768 entries for the
                same 32 rows (64 heads, d=128) in GB/s against HBM peak;
  multilayer    one refresh of a three-layer threshold selection with OR-union
                at the decode shape, in GB/s of indexer keys against HBM peak,
                and a three-layer stack with previous-layer reuse (indexer
                top-k plus sparse attention per layer);
  projection    the query projection that produces the prefill workload's q
                (S=16384, r=2048 -> 64 x 128) in TFLOP/s against bf16 peak;
  cpu_baseline  the fp64 CPU oracle timed on a bounded sample of the same rows.

    python bench.py [--gpus 1] [--steps 100] [--warmup 50]
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "indexer TFLOP/s (% bf16 MFMA peak) prefill; decode key-scan GB/s (% HBM peak)"


def _log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _to_dev(p, torch, dev):
    import numpy as np
    if p["dtype"] == "bf16":
        q = torch.from_numpy(p["q"].view(np.int16)).view(torch.bfloat16)
        k = torch.from_numpy(p["k"].view(np.int16)).view(torch.bfloat16)
    else:
        q, k = torch.from_numpy(p["q"]), torch.from_numpy(p["k"])
    return q.to(dev), k.to(dev), torch.from_numpy(p["w"]).to(dev)


def _time_calls(torch, call, steps, warmup):
    """Warm up, then time exactly `steps` back-to-back calls between two HIP
    events on the current stream (the timed region).  Per-launch durations
    come from a second pass of `steps` calls, each bracketed by its own event
    pair: an event recorded between two calls leaves the GPU idle for a few
    microseconds, so those events stay out of the timed region."""
    for i in range(warmup):
        call(i)
    st = torch.cuda.current_stream()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(st)
    for i in range(steps):
        call(i)
    t1.record(st)
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record(st)
        call(i)
        ev[i][1].record(st)
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) for a, b in ev)
    return total_ms, sum(per) / len(per), per[len(per) // 2], per[0]


def kernel_source_sha256():
    """sha256 over the device sources (kernels and the headers they include),
    in a fixed order: a traffic record applies only to the source it was
    measured on."""
    h = hashlib.sha256()
    for f in ("csa_kernels.hip", "csa_device.hpp", "csa_internal.hpp"):
        h.update(open(os.path.join(ROOT, "lightning_indexer_top_02_amd", "csrc", f), "rb").read())
    return h.hexdigest()


def _traffic_record(kernel):
    """HBM bytes per launch measured by rocprofv3 counters, if recorded for the
    current kernel source (null once the kernel source changes)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path)).get(kernel)
        sha = kernel_source_sha256()
        if rec and rec.get("src_sha256") == sha:
            return rec
    except (OSError, ValueError):
        pass
    return None


def bench_prefill(args, torch, L, csa_inputs, R, cfg=2):
    dev = torch.device("cuda:0")
    p = csa_inputs.config(cfg)
    q, k, w = _to_dev(p, torch, dev)
    topk = p["topk"]
    prob = L.make_problem(q, k, w, m=p["m"], q_pos0=p["q_pos0"])
    lib = L.load_library()
    out = torch.empty((p["B"], p["S_q"], topk), dtype=torch.int32, device=dev)
    nws = L.workspace_size(L.OP_PREFILL, prob, topk)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    pb = ctypes.byref(prob)
    op, wp = ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(ws.data_ptr())

    def call(_):
        s = lib.csa_index_topk_prefill(pb, topk, 0, op, None, wp, nws, stream)
        if s != 0:
            raise RuntimeError(lib.csa_last_error().decode())

    need, allv = R.visible_pairs(p["S_q"], p["q_pos0"], p["m"], p["T"], topk)
    flops = R.prefill_flops(p["H"], p["D"], need)
    _log(f"prefill: {p['name']}; {flops / 1e9:.1f} GFLOP per step; workspace {nws / 2**20:.0f} MiB")
    total_ms, avg_ms, med_ms, min_ms = _time_calls(torch, call, args.steps, args.warmup)
    ms = total_ms / args.steps
    peak_mem = torch.cuda.max_memory_allocated(dev)
    res = dict(p=p, flops=flops, need=need, allv=allv, ms=ms, avg_ms=avg_ms, med_ms=med_ms, min_ms=min_ms,
               peak_mem=peak_mem, ws=nws)
    del q, k, w, out, ws
    torch.cuda.empty_cache()
    return res


def bench_decode(args, torch, L, csa_inputs, R):
    dev = torch.device("cuda:0")
    p = csa_inputs.config(4)
    q, k0, w = _to_dev(p, torch, dev)
    ks = [k0] + [k0.clone() for _ in range(3)]          # 4 x 256 MiB of keys rotate through
    topk = p["topk"]
    lib = L.load_library()
    probs = [L.make_problem(q, kk, w, m=p["m"], q_pos0=p["q_pos0"]) for kk in ks]
    out = torch.empty((p["B"], 1, topk), dtype=torch.int32, device=dev)
    nws = L.workspace_size(L.OP_DECODE, probs[0], topk)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    op, wp = ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(ws.data_ptr())
    refs = [ctypes.byref(pp) for pp in probs]

    def call(i):
        s = lib.csa_index_topk_decode(refs[i % 4], topk, 0, op, None, wp, nws, stream)
        if s != 0:
            raise RuntimeError(lib.csa_last_error().decode())

    nbytes = R.decode_bytes(p["B"], 1, p["T"], p["H"], p["D"], topk)
    steps = max(args.steps * 4, 40)
    total_ms, avg_ms, med_ms, min_ms = _time_calls(torch, call, steps, args.warmup)
    ms = total_ms / steps
    gbps = nbytes / (ms * 1e-3) / 1e9
    _log(f"decode: {p['name']}: {ms * 1e3:.1f} us per call, {gbps:.0f} GB/s")
    del q, ks, k0, w, out, ws
    torch.cuda.empty_cache()
    return dict(value=round(gbps, 1), unit="GB/s", ms_per_call=round(ms, 5),
                frac_hbm_peak=round(gbps / R.PEAK_HBM_GBPS, 4), bytes_per_call=nbytes,
                calls=steps, kernels_per_call=2, key_copies_rotated=4,
                workload="decode B=32 x 1 query, context 131072 (T=32768), H_I=64, d_I=128, k=2048, bf16")


def bench_attention(args, torch, L, csa_inputs, R):
    """Sparse attention over the decode workload's shape: 32 query rows, 64
    heads, 2048 selected entries per row out of T=32768 compressed key and
    value rows (bf16, d=128); K and V rotate over 4 copies (2 GiB in all) so
    the 256 MB MALL cannot hold them."""
    import numpy as np
    dev = torch.device("cuda:0")
    B, T, n_sel = 32, 32768, 2048
    p = csa_inputs.make_attention(B, 1, T, n_sel=n_sel, seed=1006)

    def bf(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)
    q, k0, v0 = bf(p["q"]), bf(p["k"]), bf(p["v"])
    idx = torch.from_numpy(p["idx"]).to(dev)
    kv = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(3)]
    lib = L.load_library()
    probs = [L.make_attn_problem(q, kk, vv) for kk, vv in kv]
    nws = L.attention_workspace_size(probs[0], n_sel)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    out = torch.empty((B, 1, 64, 128), dtype=torch.float32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    refs = [ctypes.byref(pp) for pp in probs]
    ip, op, wp = ctypes.c_void_p(idx.data_ptr()), ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(ws.data_ptr())

    def call(i):
        s = lib.csa_sparse_attention(refs[i % 4], ip, n_sel, p["scale"], op, wp, nws, stream)
        if s != 0:
            raise RuntimeError(lib.csa_last_error().decode())

    nbytes = R.attention_bytes(B, B * n_sel, 64, 128, 128, n_sel)
    steps = max(args.steps * 4, 40)
    total_ms, avg_ms, med_ms, min_ms = _time_calls(torch, call, steps, args.warmup)
    ms = total_ms / steps
    gbps = nbytes / (ms * 1e-3) / 1e9
    _log(f"attention: {ms * 1e3:.1f} us per call, {gbps:.0f} GB/s")
    del q, k0, v0, kv, idx, out, ws
    torch.cuda.empty_cache()
    return dict(value=round(gbps, 1), unit="GB/s", ms_per_call=round(ms, 5),
                frac_hbm_peak=round(gbps / R.PEAK_HBM_GBPS, 4), bytes_per_call=nbytes, calls=steps,
                kernels_per_call=2, kv_copies_rotated=4,
                workload="sparse attention B=32 x 1 query, 64 heads, d=128, 2048 of T=32768 entries, bf16")


def bench_multilayer(args, torch, L, csa_inputs, R):
    """FlashMemory-style multi-layer selection at the decode shape: three
    indexer layers (each B=32, T=32768, H_I=64, d_I=128, its own keys), a
    sigmoid-threshold selection (tau=0.5, cap 2048) per layer, OR-union of the
    three.  One refresh (what runs every 64 decode steps) is timed."""
    import numpy as np
    dev = torch.device("cuda:0")
    layers = []
    for li in range(3):
        p = csa_inputs.make_decode(seed=1007 + li, name=f"layer {li}")
        layers.append((torch.from_numpy(p["q"].view(np.int16)).view(torch.bfloat16).to(dev),
                       torch.from_numpy(p["k"].view(np.int16)).view(torch.bfloat16).to(dev),
                       torch.from_numpy(p["w"]).to(dev)))
    sel = L.MultiLayerSelector(tau=64, prob_threshold=0.5, cap=2048, union_cap=3 * 2048)

    def call(i):
        sel.select(64 * i, layers, m=p["m"], q_pos0=p["q_pos0"])     # every call is a refresh step

    nbytes = 3 * R.decode_bytes(p["B"], 1, p["T"], p["H"], p["D"], 2048)
    steps = max(args.steps, 40)
    total_ms, avg_ms, med_ms, min_ms = _time_calls(torch, call, steps, min(args.warmup, 20))
    ms = total_ms / steps
    gbps = nbytes / (ms * 1e-3) / 1e9
    _log(f"multi-layer refresh: {ms * 1e3:.1f} us per refresh, {gbps:.0f} GB/s")
    res = dict(value=round(gbps, 1), unit="GB/s", ms_per_refresh=round(ms, 5),
               frac_hbm_peak=round(gbps / R.PEAK_HBM_GBPS, 4), bytes_per_refresh=nbytes, refreshes=steps,
               refresh_interval_steps=64,
               workload="3 indexer layers x decode B=32, T=32768, H_I=64, d_I=128; threshold tau=0.5, cap 2048; "
                        "OR-union (cap 6144); the three layers selected in one batched launch")
    if not args.no_mli:
        res["previous_layer_reuse"] = _bench_mli(args, torch, L, R, layers, p)
    del layers, sel
    torch.cuda.empty_cache()
    return res


def _bench_mli(args, torch, L, R, ind_layers, p):
    """Previous-layer reuse over the same three indexer layers, each with its
    own attention K/V (B=32, T=32768, 64 heads, d=128, top-2048): layer 0 runs
    its indexer then attends; layer 1 attends over layer 0's selection while
    layer 1's indexer runs (for layer 2); layer 2 attends over layer 1's.
    Timed on one stream and with the indexer on a second stream."""
    g = torch.Generator(device="cuda").manual_seed(1010)
    layers = []
    for ind in ind_layers:
        B, T = ind[1].shape[0], ind[1].shape[1]
        att = tuple(torch.randn(shape, device="cuda", generator=g).to(torch.bfloat16)
                    for shape in ((B, 1, 64, 128), (B, T, 128), (B, T, 128)))
        layers.append((ind, att))
    out = {}
    for ov in (False, True):
        mli = L.MultiLayerIndexer(topk=2048, overlap=ov)

        def call(_):
            mli.run(layers, m=p["m"], q_pos0=p["q_pos0"])
        total_ms, _, _, _ = _time_calls(torch, call, max(args.steps // 2, 20), min(args.warmup, 10))
        out["ms_per_stack_overlap" if ov else "ms_per_stack"] = round(total_ms / max(args.steps // 2, 20), 5)
    nbytes = 2 * R.decode_bytes(p["B"], 1, p["T"], p["H"], p["D"], 2048) + \
        3 * R.attention_bytes(p["B"], p["B"] * 2048, 64, 128, 128, 2048)
    ms = out["ms_per_stack"]
    _log(f"previous-layer reuse, 3 layers: {ms * 1e3:.1f} us per stack (indexer on a second stream: "
         f"{out['ms_per_stack_overlap'] * 1e3:.1f} us)")
    del layers
    return dict(value=round(nbytes / (ms * 1e-3) / 1e9, 1), unit="GB/s", bytes_per_stack=nbytes,
                frac_hbm_peak=round(nbytes / (ms * 1e-3) / 1e9 / R.PEAK_HBM_GBPS, 4), **out,
                workload="3 layers: indexer top-2048 (B=32, T=32768) for layers 0 and 1, sparse attention "
                         "(64 heads, d=128) for layers 0-2 over the previous layer's selection")


def bench_projection(args, torch, L, csa_inputs, R):
    """The query projection feeding the prefill workload: S=16384 low-rank
    latents of width r=2048 -> q [16384, 64, 128] (bf16 operands, fp32
    accumulation, bf16 out), through csa_project.  MFMA-bound: 2*S*r*H*D flops."""
    import numpy as np
    dev = torch.device("cuda:0")
    S, r, H, D = 16384, 2048, 64, 128
    cb, wqb = csa_inputs.make_projection(S, H * D, r, seed=1011)
    c = torch.from_numpy(cb.view(np.int16)).view(torch.bfloat16).to(dev)
    wq = torch.from_numpy(wqb.view(np.int16)).view(torch.bfloat16).to(dev)
    y = torch.empty((S, H * D), dtype=torch.bfloat16, device=dev)
    lib = L.load_library()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    cp, wp, yp = (ctypes.c_void_p(t.data_ptr()) for t in (c, wq, y))

    def call(_):
        st = lib.csa_project(cp, wp, S, H * D, r, L.CSA_BF16, yp, stream)
        if st != 0:
            raise RuntimeError(lib.csa_last_error().decode())

    flops = 2.0 * S * r * H * D
    steps = max(args.steps // 2, 20)
    total_ms, avg_ms, med_ms, _ = _time_calls(torch, call, steps, min(args.warmup, 20))
    ms = total_ms / steps
    tf = flops / (ms * 1e-3) / 1e12
    _log(f"query projection: {ms * 1e3:.1f} us per call, {tf:.0f} TFLOP/s")
    tr = _traffic_record("project_kernel<256,256>")
    del c, wq, y
    torch.cuda.empty_cache()
    return dict(value=round(tf, 1), unit="TFLOP/s", ms_per_call=round(ms, 5),
                frac_bf16_peak=round(tf / R.PEAK_BF16_TFLOPS, 4), flops_per_call=flops, calls=steps,
                launch_ms_avg=round(avg_ms, 5), launch_ms_median=round(med_ms, 5),
                traffic=None if tr is None else tr["hbm_bytes_per_launch"],
                workload="query projection S=16384, r=2048 -> H_I*d_I=8192, bf16 in/out, fp32 accumulate")


def cpu_baseline(seconds, R):
    """Time the fp64 CPU oracle on the prefill workload: all rows when they fit
    the time budget (they do on a 16-core host: ~3 s), else a seeded sample of
    the rows that need a selection, scaled to TFLOP/s by their visible pairs."""
    import numpy as np

    import csa_inputs
    import oracle
    p = csa_inputs.config(2)
    need_rows = np.array([i for i in range(p["S_q"]) if min(i // 4 + 1, p["T"]) > p["topk"]])
    t0 = time.perf_counter()
    oracle.oracle_topk(p, rows=need_rows[-8:])           # warm-up and calibration on the longest rows
    per_row = (time.perf_counter() - t0) / 8
    if per_row * p["S_q"] <= seconds:
        rows = np.arange(p["S_q"])
        what = f"the full workload: all {p['S_q']} query rows"
    else:
        n = int(max(8, seconds / per_row))
        if n >= len(need_rows):
            rows = need_rows
            what = f"all {len(need_rows)} query rows that need a selection (the others only copy indices)"
        else:
            rows = np.sort(np.random.default_rng(77).choice(need_rows, size=n, replace=False))
            what = f"{len(rows)} seeded random rows of the {len(need_rows)} that need a selection"
    t0 = time.perf_counter()
    oracle.oracle_topk(p, rows=rows)
    dt = time.perf_counter() - t0
    pairs = sum(min(int(r) // 4 + 1, p["T"]) for r in rows if min(int(r) // 4 + 1, p["T"]) > p["topk"])
    flops = R.prefill_flops(p["H"], p["D"], pairs)
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        threads = max((i.get("num_threads") or 1) for i in info) if info else 1
    except Exception:
        threads = os.cpu_count()
    return dict(value=round(flops / dt / 1e12, 6), unit="TFLOP/s", cores=threads, kind="oracle",
                seconds=round(dt, 2),
                sample=f"{what} of the V4-Flash prefill workload ({pairs} needed visible pairs), "
                       f"fp64 numpy oracle including its top-k")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50,
                    help="untimed calls first; the GPU clock needs a few tens of ms of load to settle")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--only-decode", action="store_true")
    ap.add_argument("--no-attention", action="store_true")
    ap.add_argument("--no-multilayer", action="store_true")
    ap.add_argument("--no-mli", action="store_true", help="skip the previous-layer reuse timing")
    ap.add_argument("--no-projection", action="store_true")
    ap.add_argument("--prefill-configs", default="",
                    help="also time the prefill on these configs, e.g. 3,5 (S=65536; million-token tail)")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only copy MIB MiB device-to-device (reference for the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(query rows shard across GPUs with no exchange; see the design notes). Use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import csa_inputs
    import lightning_indexer_top_02_amd as L
    from lightning_indexer_top_02_amd import roofline as R

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    L.load_library()

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "copies": 3}), flush=True)
        return
    if args.only_decode:
        print(json.dumps(bench_decode(args, torch, L, csa_inputs, R)), flush=True)
        return
    pf = bench_prefill(args, torch, L, csa_inputs, R)
    dec = None if args.no_decode else bench_decode(args, torch, L, csa_inputs, R)
    att = None if args.no_attention else bench_attention(args, torch, L, csa_inputs, R)
    mls = None if args.no_multilayer else bench_multilayer(args, torch, L, csa_inputs, R)
    prj = None if args.no_projection else bench_projection(args, torch, L, csa_inputs, R)
    other = {}
    for cfg in [int(c) for c in args.prefill_configs.split(",") if c]:
        torch.cuda.reset_peak_memory_stats()
        save = args.steps
        args.steps = max(10, args.steps // 10)
        r = bench_prefill(args, torch, L, csa_inputs, R, cfg)
        args.steps = save
        tf = r["flops"] / (r["ms"] * 1e-3) / 1e12
        _log(f"prefill config {cfg}: {r['ms']:.3f} ms per step, {tf:.1f} TFLOP/s, peak {r['peak_mem'] / 1e9:.2f} GB")
        other[str(cfg)] = dict(workload=r["p"]["name"], ms_per_step=round(r["ms"], 4), value=round(tf, 1),
                               unit="TFLOP/s", frac_bf16_peak=round(tf / R.PEAK_BF16_TFLOPS, 4),
                               flops_per_step=r["flops"], steps=max(10, args.steps // 10),
                               peak_mem_bytes=r["peak_mem"], workspace_bytes=r["ws"],
                               materialised_score_tensor_bytes=R.materialised_score_bytes(
                                   r["p"]["B"], r["p"]["q_pos0"] + r["p"]["S_q"], r["p"]["H"], r["p"]["T"]))
    cpu = None if args.no_cpu_baseline else cpu_baseline(args.cpu_seconds, R)

    p = pf["p"]
    tflops = pf["flops"] / (pf["ms"] * 1e-3) / 1e12
    achieved = pf["flops"] / (pf["avg_ms"] * 1e-3) / 1e12
    kname = "prefill_mfma_kernel<0>"
    tr = _traffic_record(kname)
    line = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pf["ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "V4-Flash-shaped prefill: B=1, S=16384 queries, m=4, T=4096 compressed keys, "
                        "H_I=64, d_I=128, top-k=2048, causal, bf16 q/k, fp32 w",
            "B": 1, "S_q": p["S_q"], "T": p["T"], "H_I": p["H"], "d_I": p["D"], "topk": p["topk"], "m": p["m"],
            "flops_per_step": pf["flops"], "needed_pairs": pf["need"], "all_visible_pairs": pf["allv"],
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "mfma",
            "kernel": kname,
            "achieved": round(achieved, 2),
            "peak": R.PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / R.PEAK_BF16_TFLOPS, 4),
            "traffic": None if tr is None else tr["hbm_bytes_per_launch"],
            "launch_ms_avg": round(pf["avg_ms"], 5),
            "launch_ms_median": round(pf["med_ms"], 5),
            "launch_ms_min": round(pf["min_ms"], 5),
        },
        "cpu_baseline": cpu,
        "decode": dec,
        "attention": att,
        "multilayer": mls,
        "projection": prj,
        "prefill_other_configs": other or None,
        "peak_mem_bytes": pf["peak_mem"],
        "workspace_bytes": pf["ws"],
        "materialised_score_tensor_bytes": R.materialised_score_bytes(1, p["S_q"], p["H"], p["T"]),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
