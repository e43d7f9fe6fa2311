#!/usr/bin/env python3
"""Throughput of the linear resize on one MI355X.

Default workload: one RGB uint8 frame 2160 x 3840 (HWC) resized linearly to
1080 x 1920 - the 4K -> 1080p case.  A step is one resize_linear call over one
frame.  Inputs are seeded synthetic frames (smooth gradients + noise) already
resident in HBM; the step rotates over enough (src, dst) buffer pairs that
their total exceeds twice the 256 MB Infinity Cache, so each step reads its
source from HBM, not from cache.

Prints ONE JSON line with: Gpix/s (dst pixels per second, whole job), the
kernel's HBM roofline (algorithmic bytes = src read once + dst written once,
over the kernel's average duration measured with HIP events on the launch
stream), and the CPU oracle timed on the host cores as a reported baseline.

    python bench.py [--steps K] [--warmup W] [--workload 4k] [--no-cpu]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0            # MI355X HBM3E, published peak
INFINITY_CACHE_BYTES = 256 << 20  # MI355X last-level (MALL) cache

# HBM bytes per launch from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE (KiB per
# dispatch), each scaled by the factor the same counter reads for the plain
# 16-byte copy of 32 MiB (`bench.py --copy-calibration 33554432`: FETCH_SIZE
# 16390.74 KiB -> x 1.9992, WRITE_SIZE 32798.97 KiB -> x 0.9991).  Valid only
# for the kernel named; profiles/linear_half_u8_4k_rgb_pmc_traffic.md holds
# the runs.  Workloads without an entry report null.
MEASURED_TRAFFIC = {
    ("4k", "linear"): {"kernel": "linear_half_u8<3, false, false>", "fetch_kib": 12175.86, "write_kib": 6075.0,
                       "fetch_scale": 1.9992, "write_scale": 0.9991},
}


def traffic_bytes(entry):
    if not entry:
        return None
    return round((entry["fetch_kib"] * entry["fetch_scale"] + entry["write_kib"] * entry["write_scale"]) * 1024)


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=2000)
    p.add_argument("--warmup", type=int, default=200)
    p.add_argument("--workload", default="4k")
    p.add_argument("--mode", default=None, help="linear (default) or nearest")
    p.add_argument("--op", default="resize", choices=["resize", "normalize", "crop", "grey"],
                   help="normalize: the fused uint8 -> float32 resize + normalisation (NCHW, or "
                        "NHWC with --layout nhwc) "
                        "(ImageNet mean / std, alpha 1/255) on the same workload; crop: "
                        "batched crop-then-resize with seeded random-resized-crop regions")
    p.add_argument("--layout", default="nchw", choices=["nchw", "nhwc"],
                   help="output layout of --op normalize")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--warm", action="store_true", help="reuse one buffer pair (cache-resident)")
    p.add_argument("--border", default="clamp", choices=["clamp", "mirror", "wrap"],
                   help="border rule for --op resize (linear): mirror / wrap use resize_linear_border")
    p.add_argument("--graph", type=int, default=0, metavar="B",
                   help="informational: also time the steps captured B at a time into a HIP "
                        "graph and replayed (small-image latency)")
    p.add_argument("--no-trimmed", action="store_true",
                   help="skip the per-launch event timing with trimming")
    p.add_argument("--no-copy", action="store_true",
                   help="skip the copy-kernel ceiling at the same bytes per launch")
    p.add_argument("--no-pipelined", action="store_true",
                   help="skip the extra two-stream pipelined measurement")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                   help="instead of resizing, time the plain 16-byte copy kernel on BYTES "
                        "bytes (cold rotation); used to scale HBM traffic counters")
    return p.parse_args()


def copy_calibration(args):
    """Run resize_copy_bytes over `args.copy_calibration` bytes per launch,
    rotating over enough buffers to defeat the Infinity Cache."""
    import torch

    import bilinear_image_resize_amd as R

    n = args.copy_calibration
    dev = torch.device("cuda:0")
    pairs = max(2, -(-2 * INFINITY_CACHE_BYTES // (2 * n)))
    bufs = [(torch.empty(n, dtype=torch.uint8, device=dev).fill_(k & 255),
             torch.empty(n, dtype=torch.uint8, device=dev)) for k in range(pairs)]
    lib = R._load()
    sh = torch.cuda.current_stream(dev).cuda_stream
    ptrs = [(a.data_ptr(), b.data_ptr()) for a, b in bufs]
    for i in range(args.warmup):
        lib.resize_copy_bytes(ptrs[i % pairs][0], ptrs[i % pairs][1], n, sh)
    torch.cuda.synchronize(dev)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        rc = lib.resize_copy_bytes(ptrs[i % pairs][0], ptrs[i % pairs][1], n, sh)
        if rc:
            raise R.ResizeError(rc, "resize_copy_bytes")
    e1.record()
    torch.cuda.synchronize(dev)
    us = e0.elapsed_time(e1) * 1e3 / args.steps
    print(json.dumps({"copy_bytes": n, "pairs": pairs, "kernel_us": round(us, 3),
                      "GBps": round(2 * n / (us * 1e-6) / 1e9, 1)}), flush=True)


def device_hbm_peak(dev_index=0):
    """Peak HBM bandwidth from the memory interface the HIP runtime reports:
    hipDeviceGetAttribute's memory bus width (bits, attribute 59) and memory
    clock (kHz, attribute 60).  HBM3E moves 4 bits per pin per reported clock
    (its data clock runs at twice the reported one, double data rate), so
    8192 bits x 2 GHz x 4 / 8 = 8192 GB/s.  A cross-check of the published
    8 TB/s, not a replacement for it."""
    import ctypes
    try:
        hip = ctypes.CDLL("libamdhip64.so")
    except OSError:
        return None
    bus, clk = ctypes.c_int(0), ctypes.c_int(0)
    if hip.hipDeviceGetAttribute(ctypes.byref(bus), 59, dev_index) != 0:
        return None
    if hip.hipDeviceGetAttribute(ctypes.byref(clk), 60, dev_index) != 0:
        return None
    return {"bus_bits": bus.value, "mem_clock_khz": clk.value,
            "GBps_at_4_per_clock": round(4 * clk.value * 1e3 * bus.value / 8 / 1e9, 1)}


def copy_same_bytes(total_bytes, steps, lib, dev, sh):
    """A plain 16-byte copy kernel moving the same bytes per launch as one
    resize (total_bytes / 2 read + total_bytes / 2 written), over rotating
    buffers that defeat the Infinity Cache, timed like the resize."""
    import torch

    n = (total_bytes // 2 + 15) // 16 * 16
    pairs = max(2, -(-2 * INFINITY_CACHE_BYTES // (2 * n)))
    bufs = [(torch.empty(n, dtype=torch.uint8, device=dev).fill_(k & 255),
             torch.empty(n, dtype=torch.uint8, device=dev)) for k in range(pairs)]
    ptrs = [(a.data_ptr(), b.data_ptr()) for a, b in bufs]
    for i in range(2 * pairs):
        lib.resize_copy_bytes(ptrs[i % pairs][0], ptrs[i % pairs][1], n, sh)
    torch.cuda.synchronize(dev)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    bad = 0
    for i in range(steps):
        bad |= lib.resize_copy_bytes(ptrs[i % pairs][0], ptrs[i % pairs][1], n, sh)
    e1.record()
    torch.cuda.synchronize(dev)
    if bad:
        raise RuntimeError("resize_copy_bytes failed (%d)" % bad)
    us = e0.elapsed_time(e1) * 1e3 / steps
    del bufs
    return {"bytes_moved": 2 * n, "kernel_us": round(us, 3), "GBps": round(2 * n / (us * 1e-6) / 1e9, 1)}


def host_cpu_model():
    """The host CPU's model name as /proc/cpuinfo gives it ("unknown" elsewhere)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, src_np, mode, budget_s):
    """The CPU oracle as it stands, on the host cores, over whole frames of
    the same workload, repeated until about budget_s seconds have passed."""
    import oracle

    threads = max(1, min(16, os.cpu_count() or 1))
    rows_total = w.batch * w.dH
    fn = oracle.resize_linear if mode == "linear" else oracle.resize_nearest
    fn(src_np[:1], 1, 1)  # load the library outside the clock

    def one_frame():
        bounds = [rows_total * k // threads for k in range(threads + 1)]
        ts = [threading.Thread(target=fn, args=(src_np, w.dH, w.dW),
                               kwargs={"rows": (bounds[k], bounds[k + 1])})
              for k in range(threads) if bounds[k + 1] > bounds[k]]
        for t in ts:
            t.start()
        for t in ts:
            t.join()

    reps = 0
    t0 = time.perf_counter()
    while True:
        one_frame()
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    per = el / reps
    return {
        "value": round(w.dst_pixels / per / 1e9, 4),
        "unit": "Gpix/s",
        "cores": threads,
        "kind": "oracle",
        "sample": "%d whole %s frame(s), %.1f s, %.2f ms per frame, output rows split "
                  "over %d host threads of %d (%s)" % (reps, w.name, el, per * 1e3, threads,
                                                       os.cpu_count() or 1, host_cpu_model()),
    }


def cpu_single_thread(w, src_np, mode, budget_s):
    """The same oracle on one host thread, over whole frames, for about
    budget_s seconds (at least one frame)."""
    import oracle

    fn = oracle.resize_linear if mode == "linear" else oracle.resize_nearest
    reps = 0
    t0 = time.perf_counter()
    while True:
        fn(src_np, w.dH, w.dW)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    per = el / reps
    return {"value": round(w.dst_pixels / per / 1e9, 4), "unit": "Gpix/s", "cores": 1,
            "sample": "%d whole %s frame(s), %.1f s, %.2f ms per frame" % (reps, w.name, el, per * 1e3)}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the resize runs on one GPU and has no "
              "multi-GPU path (--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args)
        return

    import numpy as np
    import torch

    import bilinear_image_resize_amd as R
    from bilinear_image_resize_amd.workloads import WORKLOADS, make_source

    w = WORKLOADS[args.workload]
    mode = args.mode or w.modes[0]
    if mode not in w.modes:
        sys.exit("workload %s has no %s mode" % (w.name, mode))
    dev = torch.device("cuda:0")
    R._load()

    src_np = make_source(w)
    tdt = torch.uint8 if w.dtype == "u8" else torch.float32
    src0 = torch.from_numpy(src_np).to(dev)
    fused = args.op == "normalize"
    cropped = args.op == "crop"
    grey = args.op == "grey"
    crops_np = None
    if cropped:
        rng = np.random.default_rng(w.seed + 77)
        crops = []
        for _ in range(w.batch):   # area 8-100 %, aspect 3/4 - 4/3
            area = w.H * w.W * rng.uniform(0.08, 1.0)
            ar = np.exp(rng.uniform(np.log(3 / 4), np.log(4 / 3)))
            cw = int(min(w.W, max(1, round(np.sqrt(area * ar)))))
            ch = int(min(w.H, max(1, round(np.sqrt(area / ar)))))
            crops.append((int(rng.integers(0, w.W - cw + 1)), int(rng.integers(0, w.H - ch + 1)), cw, ch))
        crops_np = np.array(crops, dtype=np.int32)
        crops_dev = torch.from_numpy(crops_np).to(dev)
    if fused:
        if w.dtype != "u8" or mode != "linear":
            sys.exit("--op normalize needs a uint8 linear workload")
        dst_shape = (w.batch, w.C, w.dH, w.dW) if args.layout == "nchw" else (w.batch, w.dH, w.dW, w.C)
        dst_bytes = w.dst_pixels * w.C * 4
        tdt_out = torch.float32
    elif grey:
        if w.C not in (3, 4) or mode != "linear":
            sys.exit("--op grey needs an RGB(A) linear workload")
        dst_shape, dst_bytes, tdt_out = (w.batch, w.dH, w.dW, 1), w.dst_pixels * w.itemsize, tdt
    else:
        dst_shape, dst_bytes, tdt_out = w.dst_shape, w.dst_bytes, tdt
    src_bytes = w.src_bytes
    if cropped:   # only the crops are read
        src_bytes = int(sum(int(c[2]) * int(c[3]) for c in crops_np)) * w.C * w.itemsize
    pair_bytes = src_bytes + dst_bytes
    pairs = 1 if args.warm else max(2, -(-2 * INFINITY_CACHE_BYTES // pair_bytes))
    srcs = [src0] + [src0.clone() for _ in range(pairs - 1)]
    dsts = [torch.empty(dst_shape, dtype=tdt_out, device=dev) for _ in range(pairs)]
    stream = torch.cuda.current_stream(dev)
    torch.cuda.synchronize(dev)

    # Launch arguments are marshalled once; the timed loop calls the C ABI
    # entry point directly so that Python overhead stays below the kernel time.
    lib = R._load()
    entry = lib.resize_linear if mode == "linear" else lib.resize_nearest
    code = R.U8 if w.dtype == "u8" else R.F32
    if fused:
        import ctypes
        fa = ctypes.c_float * 4
        mean_c, std_c = fa(0.485, 0.456, 0.406, 0.5), fa(0.229, 0.224, 0.225, 0.25)
        base = lib.resize_linear_normalize
        layout_code = R.LAYOUTS[args.layout.upper()]

        def entry(s_, d_, N_, H_, W_, C_, code_, dH_, dW_, sh_):
            return base(s_, d_, N_, H_, W_, C_, dH_, dW_, 1.0 / 255.0, mean_c, std_c, layout_code, sh_)
    if grey:
        entry = lib.resize_linear_grey
    if args.border != "clamp":
        if mode != "linear" or fused or cropped or grey:
            sys.exit("--border applies to the plain linear resize")
        border_entry = lib.resize_linear_border
        border_code = {"mirror": 1, "wrap": 2}[args.border]

        def entry(s_, d_, N_, H_, W_, C_, code_, dH_, dW_, sh_):
            return border_entry(s_, d_, N_, H_, W_, C_, code_, dH_, dW_, border_code, sh_)
    if cropped:
        if mode != "linear":
            sys.exit("--op crop is linear only")
        roi_entry = lib.resize_linear_roi
        roi_ptr = crops_dev.data_ptr()

        def entry(s_, d_, N_, H_, W_, C_, code_, dH_, dW_, sh_):
            return roi_entry(s_, d_, N_, H_, W_, C_, code_, roi_ptr, dH_, dW_, sh_)
    sh = stream.cuda_stream
    sp = [t.data_ptr() for t in srcs]
    dp = [t.data_ptr() for t in dsts]
    N, H, W, C, dH, dW = w.batch, w.H, w.W, w.C, w.dH, w.dW

    def steps(k0, k):
        bad = 0
        for i in range(k0, k0 + k):
            j = i % pairs
            bad |= entry(sp[j], dp[j], N, H, W, C, code, dH, dW, sh)
        if bad:
            raise R.ResizeError(bad, "resize")

    steps(0, args.warmup)
    torch.cuda.synchronize(dev)

    # timed region: exactly K steps, bracketed by synchronisation, with a HIP
    # event pair on the launch stream around the whole region
    K = args.steps
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    e0.record(stream)
    steps(args.warmup, K)
    e1.record(stream)
    t_enq = time.perf_counter()
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    ker_avg_ms = e0.elapsed_time(e1) / K

    ms_per_step = wall * 1e3 / K
    gpix = w.dst_pixels / (ms_per_step * 1e-3) / 1e9
    alg_bytes = pair_bytes                    # src read once + dst written once
    achieved = alg_bytes / (ker_avg_ms * 1e-3) / 1e9

    # Informational: the same K frames with consecutive calls alternating over
    # two HIP streams (default priority), as a pipeline of independent frames
    # would issue them; one frame's launch ramp and drain overlap the next
    # frame's.  Not the headline: per-kernel durations overlap here.
    pipelined = None
    if not args.no_pipelined:
        side = [stream, torch.cuda.Stream(dev)]
        shs = [t.cuda_stream for t in side]

        def steps2(k0, k):
            bad = 0
            for i in range(k0, k0 + k):
                j = i % pairs
                bad |= entry(sp[j], dp[j], N, H, W, C, code, dH, dW, shs[i & 1])
            if bad:
                raise R.ResizeError(bad, "resize")

        steps2(0, args.warmup)
        torch.cuda.synchronize(dev)
        t0p = time.perf_counter()
        steps2(args.warmup, K)
        torch.cuda.synchronize(dev)
        wall2 = time.perf_counter() - t0p
        pipelined = {"streams": 2, "us_per_frame": round(wall2 * 1e6 / K, 3),
                     "Gpix_s": round(w.dst_pixels * K / wall2 / 1e9, 3),
                     "GBps": round(pair_bytes * K / wall2 / 1e9, 1)}

    # Informational: B steps captured once into a HIP graph and replayed, which
    # removes the per-call host cost that bounds tiny images.
    graphed = None
    if args.graph > 0:
        B = args.graph
        gstream = torch.cuda.Stream(dev)
        gstream.wait_stream(stream)
        torch.cuda.synchronize(dev)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=gstream):
            gsh = torch.cuda.current_stream(dev).cuda_stream
            for i in range(B):
                j = i % pairs
                rc = entry(sp[j], dp[j], N, H, W, C, code, dH, dW, gsh)
                if rc:
                    raise R.ResizeError(rc, "resize (capture)")
        for _ in range(3):
            graph.replay()
        torch.cuda.synchronize(dev)
        reps = max(1, K // B)
        t0g = time.perf_counter()
        for _ in range(reps):
            graph.replay()
        torch.cuda.synchronize(dev)
        wall_g = time.perf_counter() - t0g
        graphed = {"steps_per_graph": B, "replays": reps,
                   "us_per_step": round(wall_g * 1e6 / (reps * B), 3),
                   "Gpix_s": round(w.dst_pixels * reps * B / wall_g / 1e9, 3)}

    # correctness of what was timed: the last buffer written, vs the oracle
    if not args.no_cpu:
        import oracle
        got = dsts[(K - 1) % pairs].cpu().numpy()
        if cropped:
            ref = oracle.resize_linear_roi(src_np, crops_np, w.dH, w.dW)
            ok = np.array_equal(got, ref) if w.dtype == "u8" else float(np.abs(got - ref).max()) <= 1e-5
        elif grey:
            ref = oracle.resize_linear_grey(src_np, w.dH, w.dW)
            ok = np.array_equal(got, ref) if w.dtype == "u8" else float(np.abs(got - ref).max()) <= 1e-5
        elif fused:
            ref = oracle.resize_linear_normalize(src_np, w.dH, w.dW, 1 / 255, (0.485, 0.456, 0.406, 0.5)[:w.C],
                                                 (0.229, 0.224, 0.225, 0.25)[:w.C], args.layout.upper())
            ok = bool((np.abs(got - ref) <= 1e-5 * np.maximum(1.0, np.abs(ref))).all())
        else:
            if mode == "linear":
                ref = oracle.resize_linear(src_np, w.dH, w.dW, border=args.border)
            else:
                ref = oracle.resize_nearest(src_np, w.dH, w.dW)
            ok = np.array_equal(got, ref) if w.dtype == "u8" else float(np.abs(got - ref).max()) <= 1e-5
        if not ok:
            sys.exit("bench output disagrees with the oracle")

    traffic = (None if (fused or cropped or grey or args.border != "clamp")
               else traffic_bytes(MEASURED_TRAFFIC.get((w.name, mode))))
    line = {
        "metric": "bilinear resize Gpix/s + HBM GB/s (% of peak), RGB u8 4K->1080p, 1 GPU",
        "value": round(gpix, 3),
        "unit": "Gpix/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": "%s: %s %dx%dx%dx%d -> %dx%d %s%s" % (
                w.name, w.dtype, w.batch, w.H, w.W, w.C, w.dH, w.dW, mode,
                " + normalize to f32 " + args.layout.upper() if fused else (" of random crops" if cropped else
                " to grey" if grey else
                ("" if args.border == "clamp" else ", %s border" % args.border))),
            "batch": w.batch, "src_hwc": [w.H, w.W, w.C], "dst_hw": [w.dH, w.dW],
            "mode": mode, "cache": "warm (1 pair)" if args.warm else "cold (%d rotating pairs)" % pairs,
        },
        "hbm_GBps_wall": round(pair_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "kernel_us": round(ker_avg_ms * 1e3, 3),
        "host_enqueue_us": round((t_enq - t0) * 1e6 / K, 3),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
        },
    }
    # the measurement of "From Prototype to Performance" ("Measure
    # performance carefully"): launches timed one by one with HIP events,
    # sorted, 10 % trimmed at each end, averaged (informational)
    if not args.no_trimmed:
        R_ = 100
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(R_)]
        torch.cuda.synchronize(dev)
        bad = 0
        for i, (ea, eb) in enumerate(evs):
            j = i % pairs
            ea.record(stream)
            bad |= entry(sp[j], dp[j], N, H, W, C, code, dH, dW, sh)
            eb.record(stream)
        torch.cuda.synchronize(dev)
        if bad:
            raise R.ResizeError(bad, "resize")
        d = sorted(ea.elapsed_time(eb) * 1e3 for ea, eb in evs)
        cut = R_ // 10
        kept = d[cut:R_ - cut]
        line["trimmed_events"] = {"launches": R_, "trim": "10% each end",
                                  "mean_us": round(sum(kept) / len(kept), 3),
                                  "median_us": round(d[R_ // 2], 3)}
    # the copy-kernel ceiling at the same bytes per launch, and the HBM peak
    # the runtime reports (both informational)
    if not args.no_copy:
        cp = copy_same_bytes(pair_bytes, min(K, 500), R._load(), dev,
                             torch.cuda.current_stream(dev).cuda_stream)
        cp["resize_frac_of_copy"] = round(achieved / cp["GBps"], 4)
        line["copy_same_bytes"] = cp
    peak_dev = device_hbm_peak()
    if peak_dev:
        line["hbm_peak_device"] = peak_dev
    if pipelined:
        line["pipelined_two_streams"] = pipelined
    if graphed:
        line["graph_replay"] = graphed
    if not args.no_cpu and args.op == "resize":
        line["cpu_baseline"] = cpu_baseline(w, src_np, mode, args.cpu_seconds)
        line["cpu_single_thread"] = cpu_single_thread(w, src_np, mode, min(3.0, args.cpu_seconds))
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
