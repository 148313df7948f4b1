#!/usr/bin/env python3
"""Throughput of the CSA lightning-indexer top-k on one MI355X.

A step is one csa_index_topk_prefill call over the million-token tail: the
last 8192 queries of an S = 1,048,576 sequence (q_pos0 = 1,040,384) against
all T = 262,144 compressed keys (m = 4), H_I = 64, d_I = 128, top-k = 2048,
causal; bf16 q/k ~ N(0,1)/sqrt(128), fp32 w ~ N(0,1)/8; inputs resident in
HBM.  It is the largest of the workloads that fits one GPU (35.05 TFLOP per
step).  value = algorithmic TFLOP/s over the timed region: 2*H*D flops per
(query, visible key) pair over rows with more visible keys than k.

Also reported on the same JSON line:
  roofline        the prefill kernel at the headline workload against the bf16
                  MFMA peak (HIP-event time of each launch on the stream the
                  library launches on, in a pass of its own after the timed
                  region) and its counter-measured HBM traffic;
  prefill_configs the V4-Flash prefill (S=16384, T=4096) and the long prefill
                  (S=65536, T=16384), with peak device memory against the fp32
                  [S, H_I, T] score tensor the method never forms;
  interleaved     the headline workload split into 8 strided key partitions
                  (s mod 8) with a local top-320 each: time against the MFMA
                  roofline and the union's recall of the global top-2048 over
                  all 8192 rows;
  decode          the decode scan (B=32 x T=32768, k=2048) in GB/s against HBM
                  peak, K rotated over 4 copies so the 256 MB MALL cannot hold it;
  read_stream     a plain streaming read of 2 GiB: what a read-only kernel
                  reaches on this GPU (the practical ceiling of the decode scan);
  attention, multilayer, projection   the consumer of the selection, the
                  multi-layer selection policies and the query projection;
  cpu_baseline    the fp64 CPU oracle timed on a seeded sample of the
                  headline workload's rows, scaled by visible pairs.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5]

Every leg warms up for at least --min-warmup-ms of GPU work before its timed
region, whatever --warmup says: the clock needs a few hundred milliseconds of
load to settle.
"""
import argparse
import ctypes
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "indexer TFLOP/s (% bf16 MFMA peak) prefill; decode key-scan GB/s (% HBM peak)"
HEADLINE_CFG = 5
PAGES_MIN_RECALL_H200 = 0.9980       # StreamIndex abstract: min set-overlap recall, 1x H200 (context only)
PAGES_PEAK_HBM_S1M_H200 = 6.21e9     # StreamIndex abstract: peak HBM at S = 1,048,576 on 1x H200 (context only)
PREFILL_KERNEL = "prefill_mfma2_kernel<0>"  # the bf16 top-k prefill kernel the roofline is taken on


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


def _time_calls(torch, call, steps, warmup, min_warm_ms):
    """Warm up (at least `warmup` calls and at least `min_warm_ms` of wall
    time with the GPU loaded), then time exactly `steps` back-to-back calls
    between two HIP events on the current stream (the timed region).
    Per-launch durations come from a second pass of `steps` calls, each
    bracketed by its own event pair: an event recorded between two calls
    leaves the GPU idle for a few microseconds, so those events stay out of
    the timed region."""
    i = 0
    for _ in range(warmup):
        call(i)
        i += 1
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    while (time.perf_counter() - t_start) * 1e3 < min_warm_ms:
        for _ in range(4):
            call(i)
            i += 1
        torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(st)
    for _ in range(steps):
        call(i)
        i += 1
    t1.record(st)
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for j in range(steps):
        ev[j][0].record(st)
        call(i)
        i += 1
        ev[j][1].record(st)
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) for a, b in ev)
    return total_ms, sum(per) / len(per), per[len(per) // 2], per[0]


def kernel_source_sha256():
    """sha256 over the device sources (kernels and the headers they include)
    and the host code that sizes their launches and workspaces, in a fixed
    order: a traffic record applies only to the source it was measured on."""
    h = hashlib.sha256()
    for f in ("csa_kernels.hip", "csa_device.hpp", "csa_internal.hpp", "csa_api.cpp"):
        h.update(open(os.path.join(ROOT, "lightning_indexer_top_02_amd", "csrc", f), "rb").read())
    return h.hexdigest()


def _traffic_record(kernel, workload):
    """HBM bytes per launch measured by rocprofv3 counters for `kernel` on
    `workload`, if recorded for the current kernel source (null once the
    kernel source changes)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path)).get(f"{kernel} @ {workload}")
        if rec and rec.get("src_sha256") == kernel_source_sha256():
            return rec
    except (OSError, ValueError):
        pass
    return None


class PrefillCase:
    """One prefill workload resident on the device, with the C-ABI calls that
    time it (top-k, and the interleaved variant)."""

    def __init__(self, torch, L, csa_inputs, cfg):
        self.torch, self.L = torch, L
        dev = torch.device("cuda:0")
        torch.cuda.synchronize()
        torch.cuda.reset_peak_memory_stats(dev)
        self.base_mem = torch.cuda.memory_allocated(dev)
        self.p = p = csa_inputs.config(cfg)
        self.cfg = cfg
        self.q, self.k, self.w = _to_dev(p, torch, dev)
        del p["q"], p["k"]                          # host copies are no longer needed
        self.topk = p["topk"]
        self.prob = L.make_problem(self.q, self.k, self.w, m=p["m"], q_pos0=p["q_pos0"])
        self.lib = L.load_library()
        self.out = torch.empty((p["B"], p["S_q"], self.topk), dtype=torch.int32, device=dev)
        self.nws = L.workspace_size(L.OP_PREFILL, self.prob, self.topk)
        self.ws = torch.empty(self.nws, dtype=torch.uint8, device=dev)
        self.stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def topk_call(self):
        lib, pb, topk, nws, stream = self.lib, ctypes.byref(self.prob), self.topk, self.nws, self.stream
        op, wp = ctypes.c_void_p(self.out.data_ptr()), ctypes.c_void_p(self.ws.data_ptr())

        def call(_):
            s = lib.csa_index_topk_prefill(pb, topk, 0, op, None, wp, nws, stream)
            if s != 0:
                raise RuntimeError(lib.csa_last_error().decode())
        return call

    def free(self):
        for n in ("q", "k", "w", "out", "ws"):
            setattr(self, n, None)
        self.torch.cuda.empty_cache()


def bench_prefill(args, torch, L, csa_inputs, R, cfg, steps, keep=False):
    c = PrefillCase(torch, L, csa_inputs, cfg)
    p = c.p
    need, allv = R.visible_pairs(p["S_q"], p["q_pos0"], p["m"], p["T"], c.topk)
    flops = R.prefill_flops(p["H"], p["D"], need)
    _log(f"prefill config {cfg}: {p['name']}; {flops / 1e12:.3f} TFLOP per step; workspace {c.nws / 2**20:.0f} MiB")
    total_ms, avg_ms, med_ms, min_ms = _time_calls(torch, c.topk_call(), steps, args.warmup, args.min_warmup_ms)
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated() - c.base_mem
    ms = total_ms / steps
    tf = flops / (ms * 1e-3) / 1e12
    _log(f"  {ms:.3f} ms per step, {tf:.1f} TFLOP/s ({tf / R.PEAK_BF16_TFLOPS:.1%} of bf16 peak); "
         f"per launch {avg_ms:.3f} ms; peak device memory {peak / 1e9:.2f} GB")
    res = dict(case=c, p=p, flops=flops, need=need, allv=allv, ms=ms, avg_ms=avg_ms, med_ms=med_ms,
               min_ms=min_ms, peak_mem=peak, ws=c.nws, steps=steps)
    if not keep:
        c.free()
        res["case"] = None
    return res


def _forbidden_bytes(p, R):
    """The fp32 [B, S_q, H_I, T] score tensor of this workload's query rows."""
    return R.materialised_score_bytes(p["B"], p["S_q"], p["H"], p["T"])


def prefill_summary(r, R):
    p = r["p"]
    tf = r["flops"] / (r["ms"] * 1e-3) / 1e12
    ach = r["flops"] / (r["avg_ms"] * 1e-3) / 1e12
    return dict(workload=p["name"], ms_per_step=round(r["ms"], 5), value=round(tf, 1), unit="TFLOP/s",
                frac_bf16_peak=round(tf / R.PEAK_BF16_TFLOPS, 4), steps=r["steps"],
                launch_ms_avg=round(r["avg_ms"], 5), launch_frac_bf16_peak=round(ach / R.PEAK_BF16_TFLOPS, 4),
                flops_per_step=r["flops"], needed_pairs=r["need"], all_visible_pairs=r["allv"],
                peak_mem_bytes=r["peak_mem"], workspace_bytes=r["ws"],
                materialised_score_tensor_bytes=_forbidden_bytes(p, R),
                peak_mem_frac_of_materialised=round(r["peak_mem"] / _forbidden_bytes(p, R), 6))


def bench_interleaved(args, torch, L, R, hl, P=8, k_local=320):
    """The headline workload with its keys split into P strided partitions
    (s mod P), a local top-k_local each: time per call against the MFMA
    roofline, and the union's recall of the global top-k (the headline
    call's output) over every query row."""
    c = hl["case"]
    p = c.p
    lib = c.lib
    dev = c.q.device
    out = torch.empty((p["B"], p["S_q"], P * k_local), dtype=torch.int32, device=dev)
    nws = L.workspace_size(L.OP_INTERLEAVED, c.prob, k_local, P)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    pb, op, wp = ctypes.byref(c.prob), ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(ws.data_ptr())

    def call(_):
        s = lib.csa_index_topk_interleaved(pb, P, k_local, 0, op, None, wp, nws, c.stream)
        if s != 0:
            raise RuntimeError(lib.csa_last_error().decode())

    steps = max(3, args.steps // 2)
    total_ms, avg_ms, _, _ = _time_calls(torch, call, steps, 1, args.min_warmup_ms / 2)
    ms = total_ms / steps
    pairs = R.interleaved_pairs(p["S_q"], p["q_pos0"], p["m"], p["T"], P, k_local)
    flops = R.prefill_flops(p["H"], p["D"], pairs)
    tf = flops / (ms * 1e-3) / 1e12
    # recall of the union against the global top-k (c.out holds the headline call's result)
    glob = c.out
    rec = L.set_recall(out, glob, p["T"])
    part = torch.remainder(glob.view(-1, glob.shape[-1]).long(), P)
    cnt = torch.zeros((part.shape[0], P), dtype=torch.int64, device=dev)
    cnt.scatter_add_(1, part, torch.ones_like(part))
    closed = torch.clamp(cnt, max=k_local).sum(1).double() / glob.shape[-1]
    torch.cuda.synchronize()
    rec_c = rec.double().cpu()
    closed_c = closed.cpu()
    dropped = int((cnt > k_local).sum().item())
    res = dict(workload=f"{p['name']}, P={P} strided partitions (s mod {P}), local top-{k_local} each",
               ms_per_call=round(ms, 5), value=round(tf, 1), unit="TFLOP/s",
               frac_bf16_peak=round(tf / R.PEAK_BF16_TFLOPS, 4), launch_ms_avg=round(avg_ms, 5),
               flops_per_call=flops, calls=steps, rows=int(rec_c.numel()),
               recall_mean=round(float(rec_c.mean()), 7), recall_min=round(float(rec_c.min()), 6),
               rows_below_1=int((rec_c < 1).sum()), row_partitions=int(cnt.numel()),
               row_partitions_dropping=dropped, max_partition_share=int(cnt.max().item()),
               recall_equals_closed_form=bool((rec_c.float() == closed_c.float()).all()),
               pages_min_recall_h200=PAGES_MIN_RECALL_H200,
               note="recall = |union of local top-320s ∩ global top-2048| / 2048 per row (csa_set_recall); "
                    "closed form sum_p min(c_p, 320)/2048 with c_p = global top-k members in partition p; "
                    "the pages' 0.9980 is StreamIndex's min recall on an H200, context only")
    _log(f"interleaved P={P} k_local={k_local}: {ms:.3f} ms per call, {tf:.1f} TFLOP/s; recall mean "
         f"{res['recall_mean']} min {res['recall_min']}; {dropped} of {cnt.numel()} row-partitions drop indices")
    del out, ws
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
    ws = torch.zeros(nws, dtype=torch.uint8, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    op, wp = ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(ws.data_ptr())
    refs = [ctypes.byref(pp) for pp in probs]

    def call(i):
        s = lib.csa_index_topk_decode(refs[i % 4], topk, 0, op, None, wp, nws, stream)
        if s != 0:
            raise RuntimeError(lib.csa_last_error().decode())

    nbytes = R.decode_bytes(p["B"], 1, p["T"], p["H"], p["D"], topk)
    steps = max(args.steps * 4, 80)
    total_ms, avg_ms, med_ms, min_ms = _time_calls(torch, call, steps, args.warmup, args.min_warmup_ms)
    ms = total_ms / steps
    gbps = nbytes / (ms * 1e-3) / 1e9
    _log(f"decode: {p['name']}: {ms * 1e3:.1f} us per call, {gbps:.0f} GB/s ({gbps / R.PEAK_HBM_GBPS:.1%} of HBM peak)")
    split = _decode_kernel_split(torch, call, steps, nbytes, R)
    del q, ks, k0, w, out, ws
    torch.cuda.empty_cache()
    return dict(value=round(gbps, 1), unit="GB/s", ms_per_call=round(ms, 5),
                frac_hbm_peak=round(gbps / R.PEAK_HBM_GBPS, 4), bytes_per_call=nbytes,
                launch_ms_avg=round(avg_ms, 5), calls=steps, key_copies_rotated=4, kernels=split,
                workload="decode B=32 x 1 query, context 131072 (T=32768), H_I=64, d_I=128, k=2048, bf16")


def _decode_kernel_split(torch, call, calls, nbytes, R):
    """Device time of each decode kernel over `calls` back-to-back calls,
    from the HIP runtime's kernel records (torch.profiler over ROCTracer),
    and the key scan's own rate: the algorithmic bytes of a decode call
    (keys, query, weights, output indices) over the scan kernel's average
    duration.  None if the profiler yields no records for the kernels."""
    try:
        from torch.profiler import ProfilerActivity, profile
        torch.cuda.synchronize()
        with profile(activities=[ProfilerActivity.CUDA]) as prof:
            for i in range(calls):
                call(i)
            torch.cuda.synchronize()
        dur = {}
        for e in prof.events():
            for kname in ("decode_score_kernel", "decode_select_kernel"):
                if kname in e.name:
                    dur.setdefault(kname, []).append(e.device_time_total)
        scan, sel = dur.get("decode_score_kernel"), dur.get("decode_select_kernel")
        if not scan or not sel:
            return None
        scan_us, sel_us = sum(scan) / len(scan), sum(sel) / len(sel)
        gbps = nbytes / (scan_us * 1e-6) / 1e9
        _log(f"decode kernels: key scan {scan_us:.1f} us ({gbps:.0f} GB/s, {gbps / R.PEAK_HBM_GBPS:.1%} of HBM peak), "
             f"select {sel_us:.1f} us")
        return dict(source="torch.profiler (ROCTracer) device time per kernel", calls=len(scan),
                    key_scan={"kernel": "decode_score_kernel<2048>", "us_avg": round(scan_us, 2),
                              "value": round(gbps, 1), "unit": "GB/s",
                              "frac_hbm_peak": round(gbps / R.PEAK_HBM_GBPS, 4)},
                    select={"kernel": "decode_select_kernel", "us_avg": round(sel_us, 2)})
    except Exception as exc:                          # the split is extra; the call's timing stands without it
        _log(f"decode kernel split unavailable: {exc}")
        return None


def bench_read_stream(args, torch, R):
    """A plain streaming read of 2 GiB (8x the MALL) by a read-only kernel:
    every byte loaded once with 16-byte loads, nothing written but one word
    per workgroup.  Calibrates what a read stream reaches on this GPU."""
    from lightning_indexer_top_02_amd import calib
    nbytes = 2 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1 << 16, dtype=torch.int32, device="cuda")

    def call(_):
        calib.read_stream(buf, sink)

    steps = max(args.steps, 20)
    total_ms, avg_ms, _, min_ms = _time_calls(torch, call, steps, 2, args.min_warmup_ms / 2)
    ms = total_ms / steps
    gbps = nbytes / (ms * 1e-3) / 1e9
    _log(f"read stream: {ms * 1e3:.1f} us per 2 GiB, {gbps:.0f} GB/s ({gbps / R.PEAK_HBM_GBPS:.1%} of HBM peak)")
    del buf, sink
    torch.cuda.empty_cache()
    return dict(value=round(gbps, 1), unit="GB/s", ms_per_call=round(ms, 5), bytes_per_call=nbytes,
                frac_hbm_peak=round(gbps / R.PEAK_HBM_GBPS, 4), calls=steps,
                kernel="csa_read_stream_kernel (lightning_indexer_top_02_amd/csrc/csa_calib.hip)")


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
    steps = max(args.steps * 4, 80)
    total_ms, avg_ms, med_ms, min_ms = _time_calls(torch, call, steps, args.warmup, args.min_warmup_ms / 2)
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
    total_ms, avg_ms, med_ms, min_ms = _time_calls(torch, call, steps, min(args.warmup, 20), args.min_warmup_ms / 2)
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
    steps = max(args.steps // 2, 20)
    for ov in (False, True):
        mli = L.MultiLayerIndexer(topk=2048, overlap=ov)

        def call(_):
            mli.run(layers, m=p["m"], q_pos0=p["q_pos0"])
        total_ms, _, _, _ = _time_calls(torch, call, steps, min(args.warmup, 10), args.min_warmup_ms / 4)
        out["ms_per_stack_overlap" if ov else "ms_per_stack"] = round(total_ms / steps, 5)
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
    """The query projection feeding the V4-Flash prefill: S=16384 low-rank
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
    steps = max(args.steps, 20)
    total_ms, avg_ms, med_ms, _ = _time_calls(torch, call, steps, min(args.warmup, 20), args.min_warmup_ms / 2)
    ms = total_ms / steps
    tf = flops / (ms * 1e-3) / 1e12
    _log(f"query projection: {ms * 1e3:.1f} us per call, {tf:.0f} TFLOP/s")
    tr = _traffic_record("project_kernel<256,256,2,4>", "query projection S=16384 r=2048")
    del c, wq, y
    torch.cuda.empty_cache()
    return dict(value=round(tf, 1), unit="TFLOP/s", ms_per_call=round(ms, 5),
                frac_bf16_peak=round(tf / R.PEAK_BF16_TFLOPS, 4), flops_per_call=flops, calls=steps,
                launch_ms_avg=round(avg_ms, 5), launch_ms_median=round(med_ms, 5),
                traffic=None if tr is None else tr["hbm_bytes_per_launch"],
                workload="query projection S=16384, r=2048 -> H_I*d_I=8192, bf16 in/out, fp32 accumulate")


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(seconds, R, cfg=HEADLINE_CFG):
    """Time the fp64 CPU oracle (scores and exact top-k) on a seeded sample
    of the headline workload's query rows, scaled to TFLOP/s by their visible
    pairs (2*H*D flops per pair, as for the GPU).  The sample grows until it
    takes about `seconds`: calibration on 4 rows, then one timed run."""
    import numpy as np

    import csa_inputs
    import oracle
    p = csa_inputs.config(cfg)
    vis = np.array([R.row_visible(p["q_pos0"] + i, p["m"], p["T"]) for i in range(p["S_q"])])
    need_rows = np.nonzero(vis > p["topk"])[0]
    t0 = time.perf_counter()
    oracle.oracle_topk(p, rows=need_rows[-4:])          # warm-up and calibration
    per_row = (time.perf_counter() - t0) / 4
    n = int(min(len(need_rows), max(8, seconds / per_row)))
    rows = need_rows if n >= len(need_rows) else \
        np.sort(np.random.default_rng(77).choice(need_rows, size=n, replace=False))
    t0 = time.perf_counter()
    oracle.oracle_topk(p, rows=rows)
    dt = time.perf_counter() - t0
    pairs = int(vis[rows].sum())
    flops = R.prefill_flops(p["H"], p["D"], pairs)
    total_pairs = int(vis[need_rows].sum())
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        threads = max((i.get("num_threads") or 1) for i in info) if info else 1
    except Exception:
        threads = os.cpu_count()
    return dict(value=round(flops / dt / 1e12, 6), unit="TFLOP/s", cores=threads, kind="oracle",
                seconds=round(dt, 2), cpu_model=_cpu_model(), host_cpus=os.cpu_count(),
                full_workload_seconds_extrapolated=round(dt * total_pairs / pairs, 1),
                sample=f"{len(rows)} seeded random query rows of the {len(need_rows)} of the million-token tail "
                       f"(S_q=8192, T=262144; {pairs} visible pairs), fp64 numpy oracle including its exact "
                       f"top-k; BLAS threads = cores, the per-row ReLU and head sum single-threaded numpy")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5, help="untimed calls first (at least)")
    ap.add_argument("--min-warmup-ms", type=float, default=400.0,
                    help="and at least this much wall time of untimed calls (the clock settles under load)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-attention", action="store_true")
    ap.add_argument("--no-multilayer", action="store_true")
    ap.add_argument("--no-mli", action="store_true", help="skip the previous-layer reuse timing")
    ap.add_argument("--no-projection", action="store_true")
    ap.add_argument("--no-interleaved", action="store_true")
    ap.add_argument("--no-read-stream", action="store_true")
    ap.add_argument("--prefill-configs", default="2,3",
                    help="other prefill workloads timed beside the headline (2: S=16384, 3: S=65536)")
    ap.add_argument("--only", default="", metavar="LEG",
                    help="run one leg alone and print its JSON: prefill2, prefill3, prefill5, interleaved, "
                         "decode, read, attention, multilayer, projection (for profiler runs)")
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
    if args.only:
        leg = args.only
        if leg.startswith("prefill"):
            r = bench_prefill(args, torch, L, csa_inputs, R, int(leg[7:]), args.steps)
            out = prefill_summary(r, R)
        elif leg == "interleaved":
            hl = bench_prefill(args, torch, L, csa_inputs, R, HEADLINE_CFG, 2, keep=True)
            out = bench_interleaved(args, torch, L, R, hl)
        elif leg == "decode":
            out = bench_decode(args, torch, L, csa_inputs, R)
        elif leg == "read":
            out = bench_read_stream(args, torch, R)
        elif leg == "attention":
            out = bench_attention(args, torch, L, csa_inputs, R)
        elif leg == "multilayer":
            out = bench_multilayer(args, torch, L, csa_inputs, R)
        elif leg == "projection":
            out = bench_projection(args, torch, L, csa_inputs, R)
        else:
            raise SystemExit(f"unknown leg {leg}")
        print(json.dumps(out), flush=True)
        return

    hl = bench_prefill(args, torch, L, csa_inputs, R, HEADLINE_CFG, args.steps, keep=True)
    inter = None if args.no_interleaved else bench_interleaved(args, torch, L, R, hl)
    hl["case"].free()
    hl["case"] = None
    others = {}
    for cfg in [int(c) for c in args.prefill_configs.split(",") if c]:
        r = bench_prefill(args, torch, L, csa_inputs, R, cfg, max(args.steps, 20) if cfg == 2 else args.steps)
        d = prefill_summary(r, R)
        tr = _traffic_record(PREFILL_KERNEL, r["p"]["name"])
        d["traffic"] = None if tr is None else tr["hbm_bytes_per_launch"]
        others[str(cfg)] = d
    dec = None if args.no_decode else bench_decode(args, torch, L, csa_inputs, R)
    rd = None if args.no_read_stream else bench_read_stream(args, torch, R)
    att = None if args.no_attention else bench_attention(args, torch, L, csa_inputs, R)
    mls = None if args.no_multilayer else bench_multilayer(args, torch, L, csa_inputs, R)
    prj = None if args.no_projection else bench_projection(args, torch, L, csa_inputs, R)
    cpu = None if args.no_cpu_baseline else cpu_baseline(args.cpu_seconds, R)

    p = hl["p"]
    tflops = hl["flops"] / (hl["ms"] * 1e-3) / 1e12
    achieved = hl["flops"] / (hl["avg_ms"] * 1e-3) / 1e12
    tr = _traffic_record(PREFILL_KERNEL, hl["p"]["name"])
    if dec is not None:
        tr_d = _traffic_record("decode_score_kernel<2048>", csa_inputs.config(4)["name"])
        dec["scan_traffic"] = None if tr_d is None else tr_d["hbm_bytes_per_launch"]
    line = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(hl["ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "million-token tail: the last 8192 queries of an S=1,048,576 sequence "
                        "(q_pos0=1,040,384) against T=262,144 compressed keys (m=4), H_I=64, d_I=128, "
                        "top-k=2048, causal, bf16 q/k ~ N(0,1)/sqrt(128), fp32 w ~ N(0,1)/8",
            "B": 1, "S_q": p["S_q"], "q_pos0": p["q_pos0"], "T": p["T"], "H_I": p["H"], "d_I": p["D"],
            "topk": p["topk"], "m": p["m"], "flops_per_step": hl["flops"], "needed_pairs": hl["need"],
            "all_visible_pairs": hl["allv"], "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "mfma",
            "kernel": PREFILL_KERNEL,
            "achieved": round(achieved, 2),
            "peak": R.PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / R.PEAK_BF16_TFLOPS, 4),
            "traffic": None if tr is None else tr["hbm_bytes_per_launch"],
            "launch_ms_avg": round(hl["avg_ms"], 5),
            "launch_ms_median": round(hl["med_ms"], 5),
            "launch_ms_min": round(hl["min_ms"], 5),
            "flops_per_launch": hl["flops"],
        },
        "cpu_baseline": cpu,
        "peak_mem_bytes": hl["peak_mem"],
        "workspace_bytes": hl["ws"],
        "materialised_score_tensor_bytes": _forbidden_bytes(p, R),
        "pages_peak_hbm_s1m_h200_bytes": PAGES_PEAK_HBM_S1M_H200,
        "interleaved": inter,
        "prefill_configs": others or None,
        "decode": dec,
        "read_stream": rd,
        "attention": att,
        "multilayer": mls,
        "projection": prj,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
