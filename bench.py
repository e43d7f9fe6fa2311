#!/usr/bin/env python3
"""Throughput of the linear resize on one MI355X.

Default workload: one RGB uint8 frame 2160 x 3840 (HWC) resized linearly to
1080 x 1920 - the 4K -> 1080p case.  A step is one resize_linear call over one
frame.  Inputs are seeded synthetic frames (smooth gradients + noise) already
resident in HBM; the step rotates over enough (src, dst) buffer pairs that
their total exceeds twice the 256 MB Infinity Cache, so each step reads its
source from HBM, not from cache.

Prints ONE JSON line with: Gpix/s (dst pixels per second over the K timed
steps), the kernel's HBM roofline (algorithmic bytes = src read once + dst
written once, over the kernel's average duration), and the CPU oracle timed
on the host cores as a reported baseline.

Timing protocol of the headline: the W warm-up steps are queued directly
ahead of the K timed steps, and a HIP event pair on the launch stream around
the K timed steps gives their GPU time; synchronisation brackets the region.
A bounded spin kernel (torch.cuda._sleep) holds the stream while the host
enqueues: the whole run when a step is shorter than twice the host's call
time (the GPU would otherwise outrun the host), else only the first steps.
Before any of this, untimed steps run until 50 ms of GPU work have passed
(the first milliseconds after the set-up run slower).  The steps then run
back to back as in a pipeline, starting in its steady state, and neither the
host's call rate nor its synchronisation latency enters `value`.  The wall clock of the synchronised region (hold, warm-up
and synchronisation included) is reported beside it.
`sustained` (informational) times frames issued round-robin over several
HIP streams the same way.

    python bench.py [--steps K] [--warmup W] [--workload 4k] [--no-cpu]
    python bench.py --ceiling        (launch and bandwidth ceilings)
    python bench.py --suite          (every workload, cold and warm, + oracle)
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
# dispatch), each scaled by the factor the same counter reads for a copy of
# known size (`bench.py --copy-calibration 33554432`).  Keys: (workload,
# mode).  Each entry names the profile that holds its runs and the hash of
# the kernel and launch sources it was taken on; bench.py reports null
# traffic when they no longer hash to that value (the kernel changed since).
MEASURED_TRAFFIC = {
    ("4k", "linear"): {"kernel": "linear_half_u8<3, false, false>",
                      "profile": "profiles/pmc_traffic_all_workloads.md",
                      "kernel_source_sha256_16": "1e7d296ddc1f454c",
                      "fetch_kib": 12171.034, "write_kib": 6075.0,
                      "fetch_scale": 1.99832, "write_scale": 0.99912},
    ("up2x", "linear"): {"kernel": "linear_up2_u8<1, 4, true>",
                        "profile": "profiles/pmc_traffic_all_workloads.md",
                        "kernel_source_sha256_16": "1e7d296ddc1f454c",
                        "fetch_kib": 1040.6, "write_kib": 8100.0,
                        "fetch_scale": 1.99832, "write_scale": 0.99912},
    ("thumb", "linear"): {"kernel": "rowseg<unsigned char, 3, false, 2, true, 0, false, 0, 0>",
                         "profile": "profiles/pmc_traffic_all_workloads.md",
                         "kernel_source_sha256_16": "1e7d296ddc1f454c",
                         "fetch_kib": 107575.511, "write_kib": 38592.036,
                         "fetch_scale": 1.99832, "write_scale": 0.99912},
    ("rgbaf", "linear"): {"kernel": "tile_f32<4, 1, 8, 8>",
                         "profile": "profiles/pmc_traffic_all_workloads.md",
                         "kernel_source_sha256_16": "1e7d296ddc1f454c",
                         "fetch_kib": 337077.912, "write_kib": 296628.469,
                         "fetch_scale": 1.99856, "write_scale": 0.99912},
    ("up15", "linear"): {"kernel": "tile_u8<3, 4, 16, 2, false, 0>",
                        "profile": "profiles/pmc_traffic_all_workloads.md",
                        "kernel_source_sha256_16": "1e7d296ddc1f454c",
                        "fetch_kib": 5427.929, "write_kib": 13668.751,
                        "fetch_scale": 1.99856, "write_scale": 0.99912},
}


def kernel_source_hash():
    """Hash of the kernel and launch sources (both decide what a launch does)."""
    import hashlib
    h = hashlib.sha256()
    for name in ("resize_kernels.hpp", "resize_abi.hip"):
        with open(os.path.join(ROOT, "bilinear_image_resize_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_bytes(entry):
    if not entry or entry.get("kernel_source_sha256_16") != kernel_source_hash():
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
    p.add_argument("--no-pipelined", "--no-sustained", dest="no_pipelined", action="store_true",
                   help="skip the informational multi-stream (sustained) measurement")
    p.add_argument("--hold", default="auto", choices=["auto", "whole", "first"],
                   help="stream hold of the timed run: auto (the whole run for launches shorter "
                        "than twice the host's call time, else the first 30), whole (one second, "
                        "for a tracing profiler, which slows every call), first")
    p.add_argument("--no-warm", action="store_true",
                   help="skip the informational warm-cache figure")
    p.add_argument("--streams", type=int, default=3,
                   help="HIP streams of the sustained measurement (default 3)")
    p.add_argument("--ceiling", nargs="*", default=None, metavar="SECTION",
                   help="instead of resizing, run the launch / bandwidth ceiling program "
                        "(all sections, or the ones named)")
    p.add_argument("--suite", action="store_true",
                   help="instead of one workload, measure every workload cold and warm and "
                        "time the oracle on each (single thread and all host cores)")
    p.add_argument("--copy-kind", default="library", choices=["library", "torch"],
                   help="--copy-calibration kernel: the library's 16-byte copy (non-temporal "
                        "loads and stores) or torch's tensor copy (plain loads and stores)")
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
    def one(i):
        if args.copy_kind == "torch":
            bufs[i % pairs][1].copy_(bufs[i % pairs][0])
            return
        rc = lib.resize_copy_bytes(ptrs[i % pairs][0], ptrs[i % pairs][1], n, sh)
        if rc:
            raise R.ResizeError(rc, "resize_copy_bytes")

    for i in range(args.warmup):
        one(i)
    torch.cuda.synchronize(dev)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        one(i)
    e1.record()
    torch.cuda.synchronize(dev)
    us = e0.elapsed_time(e1) * 1e3 / args.steps
    print(json.dumps({"copy_bytes": n, "copy_kind": args.copy_kind, "pairs": pairs,
                      "kernel_us": round(us, 3),
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


class StreamHold:
    """Holds a stream with torch.cuda._sleep, a bounded spin kernel, while
    the host enqueues a run of launches behind it: the HIP events around the
    run then time launches that follow each other back to back on the GPU,
    not the host's call rate.  The spin is calibrated once (clock cycles per
    microsecond) with events."""

    def __init__(self, dev, stream):
        import torch
        self.torch = torch
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            torch.cuda._sleep(1000)
            cycles = 2_000_000
            e0.record(stream)
            torch.cuda._sleep(cycles)
            e1.record(stream)
        torch.cuda.synchronize(dev)
        self.cycles_per_us = cycles / max(1e-3, e0.elapsed_time(e1) * 1e3)

    def __call__(self, stream, us):
        with self.torch.cuda.stream(stream):
            self.torch.cuda._sleep(int(us * self.cycles_per_us))


def timed_run(launch, n, streams, hold, enqueue_us, pre=None, full_hold=True, hold_us_min=0.0):
    """GPU time per launch (ms) of n launches, launch(i, stream_handle) for
    i in [0, n) on streams[i % S], timed by a HIP event pair on streams[0]
    joined with every other stream.  A bounded spin kernel first holds
    streams[0]: for the whole enqueue (full_hold: launches shorter than the
    host's call, which the GPU would otherwise outrun), or for the first 30
    (longer launches: the host stays ahead once they run, and holding a
    long queue measured up to 4 % slower for them).  `pre`, if given, is
    (launch function, count): untimed launches queued behind the hold
    directly ahead of the timed ones, on streams[0], so that the timed
    launches start in the steady state of a running queue.  Returns (ms per
    launch, host enqueue seconds, whether the hold outlasted the enqueue of
    the launches it was meant to cover)."""
    import torch
    main = streams[0]
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    n_pre = pre[1] if pre else 0
    covered = n_pre + (n if full_hold else min(n, 30))
    # about 1.5x the host's enqueue time, capped at one second (a slow host,
    # e.g. under a tracing profiler, then shows as hold_covered_enqueue false)
    hold_us = min(max(1.5 * covered * enqueue_us + 100.0, hold_us_min), 1e6)
    handles = [st.cuda_stream for st in streams]
    t0 = time.perf_counter()
    hold(main, hold_us)
    for i in range(n_pre):
        pre[0](i, handles[0])
    e0.record(main)
    for st in streams[1:]:
        st.wait_event(e0)
    for i in range(n):
        launch(i, handles[i % len(handles)])
    for st in streams[1:]:
        ev = torch.cuda.Event()
        ev.record(st)
        main.wait_event(ev)
    e1.record(main)
    t_enq = time.perf_counter() - t0
    e1.synchronize()
    return e0.elapsed_time(e1) / n, t_enq, t_enq * covered / (n + n_pre) * 1e6 < hold_us


def settle(launch, stream, min_ms=50.0, max_launches=20000):
    """Untimed launches until at least min_ms of GPU work has run.  The
    first few milliseconds of work after the set-up (buffers just written,
    the GPU idle since) run up to 20 % slower on this hardware - a 300-launch
    run of the thumbnail batch averaged 54.5 us where the next one took 45
    - so the timed launches start only after this.  Returns the launch
    count."""
    import torch
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    done, batch = 0, 8
    e0.record(stream)
    while done < max_launches:
        for i in range(batch):
            launch(done + i, stream.cuda_stream)
        done += batch
        e1.record(stream)
        e1.synchronize()
        if e0.elapsed_time(e1) >= min_ms:
            break
        batch = min(2 * batch, 512)
    return done


def needs_full_hold(launch, stream, hold, enqueue_us):
    """Whether launches are short enough (under twice the host's call time)
    that the whole timed run must be held: estimated from 12 held launches."""
    ms, _, _ = timed_run(launch, 12, [stream], hold, enqueue_us)
    return ms * 1e3 < 2.0 * enqueue_us


def copy_same_bytes(total_bytes, steps, lib, dev, stream, hold, enqueue_us):
    """A plain 16-byte copy kernel moving the same bytes per launch as one
    resize (total_bytes / 2 read + total_bytes / 2 written), over rotating
    buffers that defeat the Infinity Cache, timed like the resize (held
    stream, HIP events)."""
    import torch

    n = (total_bytes // 2 + 15) // 16 * 16
    pairs = max(2, -(-2 * INFINITY_CACHE_BYTES // (2 * n)))
    bufs = [(torch.empty(n, dtype=torch.uint8, device=dev).fill_(k & 255),
             torch.empty(n, dtype=torch.uint8, device=dev)) for k in range(pairs)]
    ptrs = [(a.data_ptr(), b.data_ptr()) for a, b in bufs]
    bad = [0]

    def launch(i, sh):
        bad[0] |= lib.resize_copy_bytes(ptrs[i % pairs][0], ptrs[i % pairs][1], n, sh)

    settle(launch, stream)
    full = needs_full_hold(launch, stream, hold, enqueue_us)
    ms, _, _ = timed_run(launch, steps, [stream], hold, enqueue_us, pre=(launch, 10),
                         full_hold=full)
    if bad[0]:
        raise RuntimeError("resize_copy_bytes failed (%d)" % bad[0])
    us = ms * 1e3
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


def ceiling(sections=None):
    """Runs the ceiling program (copy throughput against size, empty-grid
    launch costs, a read-only stream, the 4K frame on 1-4 streams, a
    per-wave trace of a stand-in for the 2:1 kernel, the exact 2x kernel
    beside stand-ins of its byte mix) and passes its JSON lines through;
    `sections` names a subset."""
    import subprocess
    exe = os.path.join(ROOT, "bilinear_image_resize_amd", "mi_resize_ceiling")
    if not os.path.exists(exe):
        sys.exit("the ceiling program is not built: run __graft_entry__.build() first")
    sys.exit(subprocess.call([exe] + list(sections or [])))


def oracle_rate(w, src_np, mode, threads, budget_s):
    """Oracle Gpix/s on `threads` host threads for about budget_s seconds.
    Each round gives every thread its own run of consecutive output rows
    (wrapping around the batch), sized to about 0.2 s of single-thread work
    from a first timed band, so thread start-up stays negligible."""
    import oracle

    fn = oracle.resize_linear if mode == "linear" else oracle.resize_nearest
    fn(src_np[:1], 1, 1)
    rows_total = w.batch * w.dH
    probe = max(1, min(rows_total, 20000 // w.dW + 1))
    t = time.perf_counter()
    fn(src_np, w.dH, w.dW, rows=(0, probe))
    s_per_row = max(1e-9, (time.perf_counter() - t) / probe)
    per = max(1, min(rows_total // threads if rows_total >= threads else 1, int(0.2 / s_per_row)))
    done, r0 = 0, 0
    t0 = time.perf_counter()
    while True:
        spans = []
        for _ in range(threads):
            if r0 >= rows_total:
                r0 = 0
            r1 = min(rows_total, r0 + per)
            spans.append((r0, r1))
            r0 = r1
        ts = [threading.Thread(target=fn, args=(src_np, w.dH, w.dW), kwargs={"rows": sp})
              for sp in spans]
        for t_ in ts:
            t_.start()
        for t_ in ts:
            t_.join()
        done += sum(b - a for a, b in spans)
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return {"Gpix_s": round(done * w.dW / el / 1e9, 5), "threads": threads,
            "sample": "%d output rows of %d, %d per thread per round (%.1f s)" % (
                done, rows_total, per, el)}


def suite(args):
    """Every workload and mode, cold (rotating buffers) and warm (one pair),
    each timed like the headline; the same-bytes copy; and the oracle on one
    host thread and on all of them (up to 16)."""
    import torch

    import bilinear_image_resize_amd as R
    from bilinear_image_resize_amd.workloads import WORKLOADS, make_source

    dev = torch.device("cuda:0")
    lib = R._load()
    stream = torch.cuda.current_stream(dev)
    hold = StreamHold(dev, stream)
    cores = max(1, min(16, os.cpu_count() or 1))
    for w in WORKLOADS.values():
        src_np = make_source(w)
        src0 = torch.from_numpy(src_np).to(dev)
        tdt = src0.dtype
        pairs = max(2, -(-2 * INFINITY_CACHE_BYTES // (w.src_bytes + w.dst_bytes)))
        srcs = [src0] + [src0.clone() for _ in range(pairs - 1)]
        dsts = [torch.empty(w.dst_shape, dtype=tdt, device=dev) for _ in range(pairs)]
        sp = [t.data_ptr() for t in srcs]
        dp = [t.data_ptr() for t in dsts]
        code = R.U8 if w.dtype == "u8" else R.F32
        for mode in w.modes:
            entry = lib.resize_linear if mode == "linear" else lib.resize_nearest
            bad = [0]

            def cold(i, sh_):
                j = i % pairs
                bad[0] |= entry(sp[j], dp[j], w.batch, w.H, w.W, w.C, code, w.dH, w.dW, sh_)

            def warm(i, sh_):
                bad[0] |= entry(sp[0], dp[0], w.batch, w.H, w.W, w.C, code, w.dH, w.dW, sh_)

            for i in range(3):
                cold(i, stream.cuda_stream)
            torch.cuda.synchronize(dev)
            t_w = time.perf_counter()
            for i in range(20):
                cold(i, stream.cuda_stream)
            enq = (time.perf_counter() - t_w) * 1e6 / 20
            torch.cuda.synchronize(dev)
            n = 300 if w.dst_pixels * w.C * w.itemsize < (64 << 20) else 100
            settle(cold, stream)
            full = needs_full_hold(cold, stream, hold, enq)
            ms_c, _, _ = timed_run(cold, n, [stream], hold, enq, pre=(cold, 10), full_hold=full)
            ms_w, _, _ = timed_run(warm, n, [stream], hold, enq, pre=(warm, 10), full_hold=full)
            if bad[0]:
                raise R.ResizeError(bad[0], "resize")
            b = w.src_bytes + w.dst_bytes
            cp = copy_same_bytes(b, n, lib, dev, stream, hold, enq)
            line = {"workload": w.name, "mode": mode, "bytes": b, "dst_pixels": w.dst_pixels,
                    "cold": {"us": round(ms_c * 1e3, 3), "GBps": round(b / ms_c / 1e6, 1),
                             "frac_of_peak": round(b / ms_c / 1e6 / HBM_PEAK_GBPS, 4),
                             "Gpix_s": round(w.dst_pixels / ms_c / 1e6, 3), "pairs": pairs},
                    "warm": {"us": round(ms_w * 1e3, 3), "GBps": round(b / ms_w / 1e6, 1),
                             "Gpix_s": round(w.dst_pixels / ms_w / 1e6, 3)},
                    "copy_same_bytes": cp}
            if not args.no_cpu:
                line["oracle_1_thread"] = oracle_rate(w, src_np, mode, 1, args.cpu_seconds / 2)
                line["oracle_all_cores"] = oracle_rate(w, src_np, mode, cores, args.cpu_seconds / 2)
                line["oracle_all_cores"]["host"] = "%d of %d threads (%s)" % (
                    cores, os.cpu_count() or 1, host_cpu_model())
            print(json.dumps(line), flush=True)
        del srcs, dsts
        torch.cuda.empty_cache()


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the resize runs on one GPU and has no "
              "multi-GPU path (--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args)
        return
    if args.ceiling is not None:
        ceiling(args.ceiling)
    if args.suite:
        suite(args)
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

    def launch(i, sh_):
        j = i % pairs
        return entry(sp[j], dp[j], N, H, W, C, code, dH, dW, sh_)

    def steps(k0, k):
        bad = 0
        for i in range(k0, k0 + k):
            bad |= launch(i, sh)
        if bad:
            raise R.ResizeError(bad, "resize")

    # first calls (library and code object loading), then the host's call rate
    steps(0, 3)
    torch.cuda.synchronize(dev)
    t_w = time.perf_counter()
    steps(3, 8)
    enqueue_us = (time.perf_counter() - t_w) * 1e6 / 8
    torch.cuda.synchronize(dev)
    hold = StreamHold(dev, stream)
    K = args.steps
    bad = [0]

    def launch_checked(i, sh_):
        bad[0] |= launch(args.warmup + i, sh_)

    def launch_warmup(i, sh_):
        bad[0] |= launch(i, sh_)

    # Warm-up, then the timed region.  The W warm-up steps are queued behind
    # the stream hold directly ahead of the K timed steps, so the timed steps
    # start in the steady state of a running queue; the HIP event pair on
    # the launch stream brackets exactly the K timed steps, and
    # synchronisation brackets the whole region.
    settled = settle(launch_warmup, stream)
    full_hold = (args.hold == "whole" or
                 (args.hold == "auto" and needs_full_hold(launch_warmup, stream, hold, enqueue_us)))
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    ker_avg_ms, t_enq, hold_ok = timed_run(launch_checked, K, [stream], hold, enqueue_us,
                                           pre=(launch_warmup, args.warmup), full_hold=full_hold,
                                           hold_us_min=1e6 if args.hold == "whole" else 0.0)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    if bad[0]:
        raise R.ResizeError(bad[0], "resize")

    ms_per_step = ker_avg_ms
    gpix = w.dst_pixels / (ms_per_step * 1e-3) / 1e9
    alg_bytes = pair_bytes                    # src read once + dst written once
    achieved = alg_bytes / (ker_avg_ms * 1e-3) / 1e9

    # Informational: frames issued round-robin over several HIP streams
    # (default priority), as a pipeline of independent frames would issue
    # them: one frame's launch ramp and drain overlap the next frame's.
    # Timed like the headline (held, HIP events, joined over the streams),
    # over at least 300 frames.  Not the headline: kernels overlap here.
    pipelined = None
    if not args.no_pipelined:
        n_s = max(K, 300)
        side = [stream] + [torch.cuda.Stream(dev) for _ in range(max(1, args.streams) - 1)]
        ms2, _, hold2 = timed_run(launch_checked, n_s, side, hold, enqueue_us)
        if bad[0]:
            raise R.ResizeError(bad[0], "resize")
        pipelined = {"streams": len(side), "frames": n_s, "us_per_frame": round(ms2 * 1e3, 3),
                     "Gpix_s": round(w.dst_pixels / (ms2 * 1e-3) / 1e9, 3),
                     "GBps": round(pair_bytes / (ms2 * 1e-3) / 1e9, 1),
                     "frac_of_peak": round(pair_bytes / (ms2 * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                     "timing": "HIP events over %d frames, streams held until all were enqueued"
                               % n_s}

    # Informational: the same launch on one buffer pair (cache-resident
    # source and destination: warm)
    warm = None
    if not args.warm and not args.no_warm:
        n_w = max(K, 300)
        def launch_warm(i, sh_):
            bad[0] |= entry(sp[0], dp[0], N, H, W, C, code, dH, dW, sh_)

        ms3, _, _ = timed_run(launch_warm, n_w, [stream], hold, enqueue_us,
                              pre=(launch_warm, 10), full_hold=full_hold)
        if bad[0]:
            raise R.ResizeError(bad[0], "resize")
        warm = {"launches": n_w, "kernel_us": round(ms3 * 1e3, 3),
                "GBps": round(pair_bytes / (ms3 * 1e-3) / 1e9, 1),
                "Gpix_s": round(w.dst_pixels / (ms3 * 1e-3) / 1e9, 3)}

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
        "timing": "HIP events around the K steps on the launch stream, held until the W warm-up "
                  "and K timed steps were enqueued (headline, roofline); wall clock of the "
                  "synchronised region beside it",
        "kernel_us": round(ker_avg_ms * 1e3, 3),
        "hbm_GBps": round(achieved, 1),
        "wall_ms_per_step": round(wall * 1e3 / K, 5),
        "host_enqueue_us": round(t_enq * 1e6 / K, 3),
        "settle_launches": settled,
        "hold": "whole run" if full_hold else "first 30 launches",
        "hold_covered_enqueue": bool(hold_ok),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
        },
    }
    entry_t = MEASURED_TRAFFIC.get((w.name, mode))
    if traffic is not None:
        line["traffic_source"] = {"profile": entry_t["profile"], "kernel": entry_t["kernel"],
                                  "counters": "rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE"}
    # the measurement of "From Prototype to Performance" ("Measure
    # performance carefully"): launches timed one by one with HIP events,
    # sorted, 10 % trimmed at each end, averaged (informational)
    if not args.no_trimmed:
        R_ = 100
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(R_)]
        torch.cuda.synchronize(dev)
        badt = 0
        for i, (ea, eb) in enumerate(evs):
            j = i % pairs
            ea.record(stream)
            badt |= entry(sp[j], dp[j], N, H, W, C, code, dH, dW, sh)
            eb.record(stream)
        torch.cuda.synchronize(dev)
        if badt:
            raise R.ResizeError(badt, "resize")
        d = sorted(ea.elapsed_time(eb) * 1e3 for ea, eb in evs)
        cut = R_ // 10
        kept = d[cut:R_ - cut]
        line["trimmed_events"] = {"launches": R_, "trim": "10% each end",
                                  "mean_us": round(sum(kept) / len(kept), 3),
                                  "median_us": round(d[R_ // 2], 3)}
    # the copy-kernel ceiling at the same bytes per launch, and the HBM peak
    # the runtime reports (both informational)
    if not args.no_copy:
        cp = copy_same_bytes(pair_bytes, max(K, 300), R._load(), dev, stream, hold, enqueue_us)
        cp["resize_frac_of_copy"] = round(achieved / cp["GBps"], 4)
        line["copy_same_bytes"] = cp
    peak_dev = device_hbm_peak()
    if peak_dev:
        line["hbm_peak_device"] = peak_dev
    if pipelined:
        line["sustained"] = pipelined
    if warm:
        line["warm"] = warm
    if graphed:
        line["graph_replay"] = graphed
    if not args.no_cpu and args.op == "resize":
        line["cpu_baseline"] = cpu_baseline(w, src_np, mode, args.cpu_seconds)
        line["cpu_single_thread"] = cpu_single_thread(w, src_np, mode, min(3.0, args.cpu_seconds))
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
