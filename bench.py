#!/usr/bin/env python3
"""Benchmark: achieved HBM GB/s of the BF16 -> MXFP4 -> block-scaled FP8 path.

A step is one pass of the whole path over one batch of synthetic input, every
launch on torch's current stream:

  for each segment (hidden 7168, intermediate 2048):
      mxfp4_quantize_rows -> mxfp4_to_fp8_rows -> mxfp4_to_fp8_cols_ragged

on the forward-chain workload (one GPU's share of a 256-expert MoE: 8 local
experts, 65536 routed rows, Zipf(1.2) counts with two empty experts).  Inputs
are resident in HBM before the timed region.  ``value`` is algorithmic bytes per
step / wall time per step.  ``roofline`` reports the dominant kernel (largest
time per step): algorithmic bytes per launch / its mean launch time, measured
with HIP events on the launch stream inside the timed region, against the
8 TB/s HBM peak.  ``per_config_scrubbed`` adds, for the dispatch workload
(32768 x 7168 over 32 experts), the weight-gradient conversion workload (quantize
and columns over 32768 x 7168, 32 experts), the dense workload (65536 x 7168) and
the forward chain, every launch's median over 20 launches each preceded by a 512 MB
scrub read (so inputs come from HBM, not the caches), next to a hand-written
16-byte streaming copy (libmxfp4bench) moving the same bytes.  ``backward`` times the FP8 gradient quantizer
(mxfp4_bf16_to_fp8_rows and mxfp4_bf16_to_fp8_cols_ragged) on the same segments,
outside ``value``, and the same quantizer writing both layouts from one read
(mxfp4_bf16_to_fp8_rows_cols_ragged); the scrubbed medians include the separate launches.  ``gemm`` times the forward expert
GEMM (mxfp4_fp8_grouped_gemm) on the hidden segment's FP8 row output against
per-expert E4M3 weights ([8, 4096, 7168], synthetic), with its MFMA roofline; ``wgrad``
times the weight-gradient GEMM (mxfp4_fp8_grouped_gemm_wgrad) on the hidden segment's
FP8 column output and a column-quantized synthetic [M, 4096] gradient; ``nvfp4`` times
the NVFP4 variant quantizer (mxfp4_nvfp4_quantize_rows, nearest even and stochastic
rounding) per forward segment.  ``cpu_baseline`` times the CPU oracle on a bounded
sample of the same workload on this host (up to 16 threads, and one thread).

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload config5] [--no-scrubbed]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "HBM GB/s & % peak: BF16→MXFP4 quant + MXFP4→FP8 row/col conversion"
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, vendor datasheet
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "block_scaled_precision_bf16tofp4row_amd", "csrc")
KERNEL_SOURCES = {
    "quantize": ["quantize.hip", "common.h"],
    "rows": ["rows.hip", "common.h"],
    "cols": ["cols.hip", "strips.h", "common.h"],
    "fp8q_rows": ["fp8q.hip", "common.h"],
    "fp8q_cols": ["fp8q_cols.hip", "strips.h", "common.h"],
    "gemm": ["gemm.hip", "strips.h", "common.h"],
    "wgrad": ["wgrad.hip", "strips.h", "common.h"],
    "nvfp4": ["nvfp4.hip", "strips.h", "common.h"],
}
FP8_MFMA_PEAK_TFLOPS = 5000.0   # MI355X dense FP8 matrix throughput, vendor datasheet
DTYPE = "bf16 -> mxfp4 (e2m1 + ue8m0 per 32) -> fp8 (e4m3fn + ue8m0 per 128)"
BENCH_LIB = os.path.join(ROOT, "block_scaled_precision_bf16tofp4row_amd", "libmxfp4bench.so")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def alg_bytes(kernel: str, M_tot: int, K: int, col_scale_bytes: int = 0) -> int:
    """Bytes the method must move (per launch)."""
    n = M_tot * K
    if kernel == "quantize":            # 2 B in, 1/2 + 1/32 B out
        return 2 * n + n // 2 + n // 32
    if kernel == "rows":                # 1/2 + 1/32 B in, 1 + 1/128 B out
        return n // 2 + n // 32 + n + n // 128
    if kernel == "cols":                # 1/2 + 1/32 B in, 1 B out + one scale byte per (block, k)
        return n // 2 + n // 32 + n + col_scale_bytes
    if kernel == "fp8q_rows":           # 2 B in, 1 + 1/128 B out
        return 2 * n + n + n // 128
    if kernel == "fp8q_cols":           # 2 B in, 1 B out + one scale byte per (block, k)
        return 2 * n + n + col_scale_bytes
    raise ValueError(kernel)


def source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(kernel: str, workload: str, segment: str):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, or None when
    there is none or the kernel source changed since the counters were taken."""
    path = os.path.join(PROFILES, f"hbm_traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"<!-- traffic-json (\{.*\}) -->", text)
    if not m:
        return None
    data = json.loads(m.group(1))
    ent = data.get(f"{kernel}/{segment}")
    if not ent or ent.get("source_sha") != source_hash(kernel):
        return None
    return ent.get("bytes_per_launch")


def affinity_cpus() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


# The oracle's thread pool: the CPUs this process may run on, at most 16 (the host
# share that goes with one GPU on a shared multi-GPU host).
MAX_ORACLE_THREADS = 16


def affinity_threads() -> int:
    return max(1, min(MAX_ORACLE_THREADS, affinity_cpus()))


# ---- CPU baseline (oracle, bounded sample) --------------------------------------------

def cpu_baseline(workload, target_s: float = 15.0):
    import oracle
    threads = affinity_threads()
    oracle._load()

    def run(rows_frac_rows):
        total_bytes = 0
        t0 = time.perf_counter()
        for seg in workload.segments:
            R = min(seg.M_tot, rows_frac_rows)
            offs = np.minimum(seg.offs, R).astype(np.int32)
            x = seg.x_bits[:R]
            c, s = oracle.quantize_rows(x, threads=threads)
            total_bytes += alg_bytes("quantize", R, seg.K)
            if "rows" in workload.kernels:
                oracle.fp8_rows(c, s, threads=threads)
                total_bytes += alg_bytes("rows", R, seg.K)
            if "cols" in workload.kernels:
                oracle.fp8_cols(c, s, offs, threads=threads)
                total_bytes += alg_bytes("cols", R, seg.K, oracle.cols_scale_size(offs, seg.K))
        return total_bytes, time.perf_counter() - t0

    probe_rows = 512
    b, t = run(probe_rows)
    max_rows = max(seg.M_tot for seg in workload.segments)
    rows = int(min(max_rows, max(probe_rows, probe_rows * target_s / max(t, 1e-6))))
    rows = max(128, rows - rows % 128)
    b, t = run(rows)
    frac = rows / max_rows
    # the plain single-threaded oracle on a smaller sample (about a third of the time)
    threads_all = threads
    threads = 1
    b1, t1 = run(probe_rows)
    rows1 = max(128, int(probe_rows * (target_s / 3) / max(t1, 1e-6)) // 128 * 128)
    rows1 = min(rows1, max_rows - max_rows % 128 or 128)
    b1, t1 = run(rows1)
    threads = threads_all
    return {
        "value": round(b / t / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "threads_used": threads,
        "affinity_cpus": affinity_cpus(),
        "kind": "oracle",
        "sample": (f"first {rows} of {max_rows} routed rows of every segment "
                   f"({frac:.1%} of a step: the same kernels, offsets clipped to the sample), "
                   f"{t:.1f} s wall on {threads} threads"),
        "single_thread": {"value": round(b1 / t1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                          "sample": f"first {rows1} routed rows of every segment, {t1:.1f} s wall"},
    }


# ---- per-kernel timing with the caches scrubbed -----------------------------------------

def build_launches(mx, workload, dev, torch, backward: bool = False):
    """Buffers and the ordered launches (kernel, segment, fn, algorithmic bytes) of one
    step of a workload: quantize -> rows -> cols per segment, as the workload lists,
    or with `backward` the FP8 gradient quantizer per segment (the segment's BF16
    tensor standing in for a gradient of the same shape)."""
    segs = []
    if backward:
        launches = []
        for seg in workload.segments:
            x = torch.from_numpy(seg.x_bits.view(np.int16)).to(dev)
            offs = torch.from_numpy(seg.offs).to(dev)
            y, ys = mx.alloc_fp8q_rows_outputs(seg.M_cap, seg.K, dev)
            yT, ysT = mx.alloc_cols_outputs(seg.M_cap, seg.K, seg.G, dev)
            nb = (np.diff(seg.offs.astype(np.int64)) + 127) // 128
            d = {"seg": seg, "x": x, "offs": offs, "y": y, "ys": ys, "yT": yT, "ysT": ysT}
            segs.append(d)
            launches.append(("fp8q_rows", seg.name,
                             lambda d=d: mx.mxfp4_bf16_to_fp8_rows(d["x"], d["y"], d["ys"], d["offs"]),
                             alg_bytes("fp8q_rows", seg.M_tot, seg.K)))
            launches.append(("fp8q_cols", seg.name,
                             lambda d=d: mx.mxfp4_bf16_to_fp8_cols_ragged(d["x"], d["yT"], d["ysT"], d["offs"]),
                             alg_bytes("fp8q_cols", seg.M_tot, seg.K, int(nb.sum()) * seg.K)))
        return segs, launches
    for seg in workload.segments:
        x = torch.from_numpy(seg.x_bits.view(np.int16)).to(dev)
        offs = torch.from_numpy(seg.offs).to(dev)
        codes, scales = mx.alloc_quantize_outputs(seg.M_cap, seg.K, dev)
        d = {"seg": seg, "x": x, "offs": offs, "codes": codes, "scales": scales}
        if "rows" in workload.kernels:
            d["y"], d["ys"] = mx.alloc_rows_outputs(seg.M_cap, seg.K, dev)
        if "cols" in workload.kernels:
            d["yT"], d["ysT"] = mx.alloc_cols_outputs(seg.M_cap, seg.K, seg.G, dev)
            nb = (np.diff(seg.offs.astype(np.int64)) + 127) // 128
            d["col_scale_bytes"] = int(nb.sum()) * seg.K
        segs.append(d)
    launches = []
    for d in segs:
        seg = d["seg"]
        launches.append(("quantize", seg.name,
                         lambda d=d: mx.mxfp4_quantize_rows(d["x"], d["codes"], d["scales"], d["offs"]),
                         alg_bytes("quantize", seg.M_tot, seg.K)))
        if "rows" in workload.kernels:
            launches.append(("rows", seg.name,
                             lambda d=d: mx.mxfp4_to_fp8_rows(d["codes"], d["scales"], d["y"], d["ys"],
                                                              d["offs"]),
                             alg_bytes("rows", seg.M_tot, seg.K)))
        if "cols" in workload.kernels:
            launches.append(("cols", seg.name,
                             lambda d=d: mx.mxfp4_to_fp8_cols_ragged(d["codes"], d["scales"], d["yT"],
                                                                     d["ysT"], d["offs"]),
                             alg_bytes("cols", seg.M_tot, seg.K, d["col_scale_bytes"])))
    return segs, launches


def scrubbed_medians(mx, torch, dev, config_ids, reps=20, warmup=5, scrub_bytes=512 << 20):
    """Per launch of each workload: median over `reps` launches, each preceded by a
    scrub that reads `scrub_bytes` (evicting the L2s and the memory-side cache, whose
    dirty lines from the previous launch are written back before the timed region,
    while the scrub's own lines are clean), timed by HIP events bound to the kernel's
    own start and end (KernelEvents); next to it the hand-written copy (bench_copy16,
    the fastest unroll measured here) moving the same number of bytes (half read, half
    written), timed the same way.  Each row also gives `median_us_markers`: the same
    launches timed by event records of their own before and after the launch on the
    stream, which add the events' commands and the dispatch gap to every launch."""
    import workloads
    stream = torch.cuda.current_stream()
    scrub = torch.ones(scrub_bytes // 4, dtype=torch.int32, device=dev)
    copy = DeviceCopy(torch, dev)
    traffic = ColsTraffic()
    kev = KernelEvents(reps)

    def median_us(fn, is_copy=False):
        """(kernel-event median, marker-event median) in microseconds."""
        for i in range(warmup):
            torch.amax(scrub)
            fn()
        for i in range(reps):
            torch.amax(scrub)
            if is_copy:
                fn(events=kev.pairs[i])
            else:
                kev.arm(mx, i)
                fn()
        k_us = float(np.median(kev.elapsed(reps)))
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in ev:
            torch.amax(scrub)
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return k_us, float(np.median([a.elapsed_time(b) for a, b in ev])) * 1000.0

    # a one-workgroup launch timed both ways: the kernel events give a trivial kernel's
    # dispatch-to-completion time, the marker events add their own share on top
    tiny_src = torch.ones(16, dtype=torch.uint8, device=dev)
    tiny_dst = torch.empty(16, dtype=torch.uint8, device=dev)
    tiny_k, tiny_m = median_us(lambda events=None: copy(tiny_dst, tiny_src, events), is_copy=True)
    log(f"[bench] scrubbed timing of a one-workgroup launch: {tiny_k:.2f} us kernel, {tiny_m:.2f} us with markers")
    out = {}
    for cid in config_ids:
        w = workloads.make_config(cid, 0)
        segs, launches = build_launches(mx, w, dev, torch)
        bsegs, blaunches = build_launches(mx, w, dev, torch, backward=True)
        launches = launches + blaunches
        for _, _, fn, _ in launches:      # valid codes for the conversions
            fn()
        torch.cuda.synchronize()
        fwd = {d["seg"].name: d for d in segs}
        bwd = {d["seg"].name: d for d in bsegs}
        rows = []
        for kern, segname, fn, nbytes in launches:
            us, us_m = median_us(fn)
            half = (nbytes // 2 + 15) // 16 * 16
            src = torch.empty(half, dtype=torch.uint8, device=dev).fill_(1)
            dst = torch.empty(half, dtype=torch.uint8, device=dev)
            cus, _ = median_us(lambda events=None: copy(dst, src, events), is_copy=True)
            del src, dst
            gbs = nbytes / (us * 1e-6) / 1e9
            copy_gbs = 2 * half / (cus * 1e-6) / 1e9
            row = {"kernel": kern, "segment": segname, "alg_bytes": nbytes,
                   "median_us": round(us, 2), "GBps": round(gbs, 1),
                   "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
                   "copy_GBps": round(copy_gbs, 1), "frac_of_copy": round(gbs / copy_gbs, 4),
                   "median_us_markers": round(us_m, 2),
                   "frac_of_peak_markers": round(nbytes / (us_m * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
            note = ""
            if kern in ("cols", "fp8q_cols"):
                d = fwd[segname] if kern == "cols" else bwd[segname]
                ceil_us, seq_us = cols_traffic_us(torch, dev, traffic, median_us, d, kern)
                row.update({"pattern_ceiling_us": round(ceil_us, 2),
                            "pattern_ceiling_frac_of_peak": round(nbytes / (ceil_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                            "frac_of_pattern_ceiling": round(ceil_us / us, 4),
                            "sequential_writes_us": round(seq_us, 2),
                            "sequential_writes_frac_of_peak": round(nbytes / (seq_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)})
                note = (f"; memory-only traffic {ceil_us:.1f} us ({row['pattern_ceiling_frac_of_peak']:.1%} of peak, "
                        f"kernel at {ceil_us / us:.1%} of it), same reads with sequential writes {seq_us:.1f} us "
                        f"({row['sequential_writes_frac_of_peak']:.1%})")
            rows.append(row)
            log(f"[bench] scrubbed {w.name} {kern}/{segname}: {us:.1f} us ({us_m:.1f} with markers), "
                f"{gbs:.0f} GB/s ({gbs / HBM_PEAK_GBS:.1%} of peak, {gbs / copy_gbs:.1%} of a same-size copy){note}")
        out[w.name] = rows
        del segs, launches, bsegs, blaunches
        torch.cuda.empty_cache()
    del scrub
    kev.close()
    torch.cuda.empty_cache()
    out["copy_kernel"] = {"what": "bench_copy16: 16-byte nontemporal loads then stores, one-shot grid",
                          "unroll": copy.unroll, "unroll_GBps_1GiB": copy.sweep}
    out["pattern_ceiling"] = {"what": "bench_cols_traffic: the column kernel's loads and whole-line stores of each "
                                      "(256-column tile, 128-row strip) on the launch's own ragged layout, one "
                                      "workgroup per pair, tile by tile over consecutive strips, no conversion, LDS or "
                                      "synchronisation (a memory-only ceiling for this traffic)",
                              "sequential_writes": "the same loads, each workgroup's stores to one contiguous 32 KB "
                                                   "block instead of the transposed columns"}
    out["timing"] = {"median_us": "HIP events bound to the kernels' own start and end (hipExtLaunchKernel "
                                  "through mxfp4_time_next_launch; the copy's own event arguments)",
                     "median_us_markers": "HIP event records before and after the launch on its stream",
                     "one_workgroup_launch_us": round(tiny_k, 2),
                     "one_workgroup_launch_us_markers": round(tiny_m, 2)}
    return out


def strip_table(offs, K: int):
    """int64 [strips, 4] of a ragged segment, in expert order: first row, rows, output byte
    of (column 0, the strip's first row) in the transposed layout, the expert's rows."""
    rows = []
    offs = np.asarray(offs, dtype=np.int64)
    for g in range(len(offs) - 1):
        r0, mg = int(offs[g]), int(offs[g + 1] - offs[g])
        for b in range((mg + 127) // 128):
            rows.append((r0 + 128 * b, min(128, mg - 128 * b), K * r0 + 128 * b, mg))
    return np.array(rows, dtype=np.int64).reshape(-1, 4)


class ColsTraffic:
    """bench_cols_traffic of libmxfp4bench: the memory-only traffic of a column kernel."""

    def __init__(self):
        import ctypes
        self.lib = DeviceCopy.load()
        P, I64 = ctypes.c_void_p, ctypes.c_int64
        self.lib.bench_cols_traffic.argtypes = [P, I64, ctypes.c_int, P, I64, P, I64, P, P, I64, I64,
                                                ctypes.c_int, P, P, P]
        self.lib.bench_cols_traffic.restype = ctypes.c_int

    def __call__(self, torch, inp, tile_in_bytes, sc, out, out_scales, strips, K, sequential, events=None):
        start, stop = events if events else (None, None)
        n = strips.shape[0]
        st = self.lib.bench_cols_traffic(
            inp.data_ptr(), inp.shape[1] * inp.element_size(), tile_in_bytes,
            sc.data_ptr() if sc is not None else None, sc.shape[1] if sc is not None else 0,
            out.data_ptr(), out.numel() * out.element_size(), out_scales.data_ptr(), strips.data_ptr(), n, K,
            1 if sequential else 0, torch.cuda.current_stream().cuda_stream, start, stop)
        if st != 0:
            raise RuntimeError(f"bench_cols_traffic failed: {st}")


def cols_traffic_us(torch, dev, traffic, median_us, d, kern):
    """Scrubbed medians (us) of the memory-only traffic of a column launch over segment
    buffers d: in the transposed layout, and with sequential writes."""
    seg = d["seg"]
    K = seg.K
    strips = torch.from_numpy(strip_table(seg.offs, K)).to(dev)
    n = strips.shape[0]
    if n == 0:
        return float("nan"), float("nan")
    if kern == "cols":
        inp, tib, sc = d["codes"], 128, d["scales"]
    else:
        inp, tib, sc = d["x"], 512, None
    out_scales = torch.empty(n * K, dtype=torch.uint8, device=dev)
    ceil_us, _ = median_us(lambda events=None: traffic(torch, inp, tib, sc, d["yT"], out_scales, strips, K, False,
                                                       events), is_copy=True)
    nkt = (K + 255) // 256
    seq_out = torch.empty(nkt * n * 256 * 128, dtype=torch.uint8, device=dev)
    seq_us, _ = median_us(lambda events=None: traffic(torch, inp, tib, sc, seq_out, out_scales, strips, K, True,
                                                      events), is_copy=True)
    del seq_out, out_scales, strips
    return ceil_us, seq_us


class KernelEvents:
    """Pairs of HIP events (libmxfp4bench) bound by the launches themselves to their
    kernels' start and end: the conversion library's timing hook
    (mxfp4_time_next_launch) arms them for the next call, the copy kernel takes them as
    arguments.  Their elapsed time is the kernels' execution, as a kernel trace reports
    it, and no event commands of their own go on the stream between launches."""

    def __init__(self, n):
        self.lib = DeviceCopy.load()
        self.pairs = [(self.lib.bench_event_create(), self.lib.bench_event_create()) for _ in range(n)]
        if not all(a and b for a, b in self.pairs):
            raise RuntimeError("hipEventCreate failed")

    def arm(self, mx, i):
        mx.mxfp4_time_next_launch(*self.pairs[i])

    def elapsed(self, n=None):
        """Microseconds of pairs 0..n-1 (waits for each stop event)."""
        out = []
        for a, b in self.pairs[: len(self.pairs) if n is None else n]:
            us = self.lib.bench_event_elapsed_us(a, b)
            if us < 0:
                raise RuntimeError("a timing event was not recorded by its launch")
            out.append(us)
        return out

    def close(self):
        for a, b in self.pairs:
            self.lib.bench_event_destroy(a)
            self.lib.bench_event_destroy(b)
        self.pairs = []


class DeviceCopy:
    """The hand-written streaming copy of libmxfp4bench, with the unroll (16-byte pieces
    per thread) that moves 1 GiB fastest on this GPU."""

    @staticmethod
    def load():
        import ctypes
        if not os.path.exists(BENCH_LIB):
            raise RuntimeError(f"{BENCH_LIB} is missing: build with "
                               "`python -m block_scaled_precision_bf16tofp4row_amd.build`")
        lib = ctypes.CDLL(BENCH_LIB)
        P = ctypes.c_void_p
        lib.bench_copy16.argtypes = [P, P, ctypes.c_int64, ctypes.c_int, P, P, P]
        lib.bench_copy16.restype = ctypes.c_int
        lib.bench_event_create.argtypes = []
        lib.bench_event_create.restype = P
        lib.bench_event_destroy.argtypes = [P]
        lib.bench_event_destroy.restype = None
        lib.bench_event_elapsed_us.argtypes = [P, P]
        lib.bench_event_elapsed_us.restype = ctypes.c_double
        return lib

    def __init__(self, torch, dev):
        self.torch = torch
        self.lib = self.load()
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty(n, dtype=torch.uint8, device=dev)
        self.sweep = {}
        for u in (1, 2, 4, 8):
            self.unroll = u
            for _ in range(3):
                self(dst, src)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(10):
                self(dst, src)
            b.record()
            torch.cuda.synchronize()
            self.sweep[u] = round(2 * n * 10 / (a.elapsed_time(b) * 1e-3) / 1e9, 1)
        assert torch.equal(dst[:: 1 << 20], src[:: 1 << 20])
        self.unroll = max(self.sweep, key=self.sweep.get)
        log(f"[bench] copy kernel GB/s by unroll (1 GiB): {self.sweep}; using {self.unroll}")
        del src, dst

    def __call__(self, dst, src, events=None):
        n = min(dst.numel() * dst.element_size(), src.numel() * src.element_size())
        start, stop = events if events else (None, None)
        st = self.lib.bench_copy16(dst.data_ptr(), src.data_ptr(), n // 16, self.unroll,
                                   self.torch.cuda.current_stream().cuda_stream, start, stop)
        if st != 0:
            raise RuntimeError(f"bench_copy16 failed: {st}")


# ---- GPU run -----------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="config5", choices=["config2", "config3", "config4", "config5"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain device copy of known size (for HBM counter scaling)")
    ap.add_argument("--gemm-n", type=int, default=4096,
                    help="output features of the expert GEMM timed on the hidden segment (0: skip)")
    ap.add_argument("--no-scrubbed", action="store_true",
                    help="skip the per-kernel scrubbed medians of configs 2, 3, 4 and 5")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the path shards by rows and "
              f"experts across GPUs (one process per GPU, each running this single-GPU path on its share), "
              f"but this benchmark measures one GPU's share.", file=sys.stderr)
        sys.exit(2)

    import torch
    import block_scaled_precision_bf16tofp4row_amd as mx
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    mx.load_library()
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)

    t0 = time.perf_counter()
    w = workloads.make_config(int(args.workload[-1]), 0)
    log(f"[bench] generated {w.name} in {time.perf_counter() - t0:.1f}s: {w.description}")

    segs, launches = build_launches(mx, w, dev, torch)   # (kernel, segment, fn, alg bytes)
    torch.cuda.synchronize()
    step_bytes = sum(l[3] for l in launches)

    nl = len(launches)

    def step(kev=None, s=0, only=None):
        """One pass of the chain; with `kev`, launch i of step s is timed by event pair
        s * nl + i (only launch `only` when given)."""
        for i, (_, _, fn, _) in enumerate(launches):
            if kev is not None and (only is None or i == only):
                kev.arm(mx, s * nl + i)
            fn()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # per-launch means from an untimed pass with every launch timed; the timed region
    # then times only the dominant launch (the events are bound to the kernels, so the
    # timing puts no commands of its own between the launches either way)
    kev = KernelEvents(args.steps * nl)
    for s in range(args.steps):
        step(kev, s)
    pus = kev.elapsed()
    per_kernel = []
    for i, (kern, segname, _, nbytes) in enumerate(launches):
        ms = [pus[s * nl + i] / 1000.0 for s in range(args.steps)]
        mean_ms = float(np.mean(ms))
        per_kernel.append({
            "kernel": kern, "segment": segname, "alg_bytes": nbytes,
            "mean_us": round(mean_ms * 1000.0, 2), "median_us": round(float(np.median(ms)) * 1000.0, 2),
            "GBps": round(nbytes / (mean_ms / 1000.0) / 1e9, 1),
            "frac_of_peak": round(nbytes / (mean_ms / 1000.0) / 1e9 / HBM_PEAK_GBS, 4),
        })
    dom_i = max(range(len(per_kernel)), key=lambda i: per_kernel[i]["mean_us"])

    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for s in range(args.steps):
        step(kev, s, only=dom_i)
    torch.cuda.synchronize()
    t_end = time.perf_counter()
    ms_per_step = (t_end - t_start) * 1000.0 / args.steps

    # the dominant launch as measured inside the timed region
    dus = kev.elapsed()
    dms = [dus[s * nl + dom_i] / 1000.0 for s in range(args.steps)]
    kev.close()
    d_mean = float(np.mean(dms))
    dnb = per_kernel[dom_i]["alg_bytes"]
    dom = dict(per_kernel[dom_i])
    dom.update({"mean_us": round(d_mean * 1000.0, 2), "GBps": round(dnb / (d_mean / 1000.0) / 1e9, 1)})
    achieved = dom["GBps"]
    traffic = read_traffic(dom["kernel"], w.name, dom["segment"])

    def time_launches(fn):
        """Milliseconds per call of `fn` (one entry-point call), kernel events."""
        for _ in range(max(1, args.warmup)):
            fn()
        tev = KernelEvents(args.steps)
        torch.cuda.synchronize()
        for i in range(args.steps):
            tev.arm(mx, i)
            fn()
        ms = [us / 1000.0 for us in tev.elapsed()]
        tev.close()
        return ms

    def mfma_entry(what, shape, flop, ms):
        us = float(np.mean(ms)) * 1000.0
        tflops = flop / (us * 1e-6) / 1e12
        log(f"[bench] {what}: {us:.1f} us, {tflops:.0f} TFLOP/s ({tflops / FP8_MFMA_PEAK_TFLOPS:.1%} of the FP8 peak)")
        return {
            "what": what, "shape": shape, "flop_per_launch": flop,
            "mean_us": round(us, 2), "median_us": round(float(np.median(ms)) * 1000.0, 2),
            "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": FP8_MFMA_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tflops / FP8_MFMA_PEAK_TFLOPS, 4)},
        }

    # the forward expert GEMM on the hidden segment's FP8 row output (not in `value`)
    gemm = None
    if args.gemm_n > 0 and "y" in segs[0]:
        seg0 = segs[0]
        sg = seg0["seg"]
        Ng, Kg, Gg = int(args.gemm_n), sg.K, sg.G
        gen = torch.Generator(device=dev)
        gen.manual_seed(0)
        wq = torch.randint(0, 256, (Gg, Ng, Kg), device=dev, dtype=torch.int32, generator=gen)
        wq = torch.where((wq & 0x7F) == 0x7F, wq - 1, wq).to(torch.uint8)        # no NaN bytes
        wqs = torch.randint(118, 136, (Gg, Ng, Kg // 128), device=dev, dtype=torch.int32, generator=gen).to(torch.uint8)
        yg = torch.empty((sg.M_cap, Ng), dtype=torch.int16, device=dev)
        gms = time_launches(lambda: mx.mxfp4_fp8_grouped_gemm(seg0["y"], seg0["ys"], wq, wqs, yg, seg0["offs"]))
        gemm = mfma_entry("forward expert GEMM: hidden-segment FP8 row output x per-expert E4M3 weights -> BF16",
                          {"M_tot": sg.M_tot, "K": Kg, "N": Ng, "G": Gg}, 2.0 * sg.M_tot * Ng * Kg, gms)
        del wq, wqs, yg

    # the weight-gradient GEMM on the hidden segment's FP8 column output and the column
    # quantization of a synthetic [M_cap, N] BF16 gradient (not in `value`)
    wgrad = None
    if args.gemm_n > 0 and "yT" in segs[0]:
        seg0 = segs[0]
        sg = seg0["seg"]
        Ng, Kg, Gg = int(args.gemm_n), sg.K, sg.G
        gen = torch.Generator(device=dev)
        gen.manual_seed(1)
        grad = (torch.randn((sg.M_cap, Ng), device=dev, generator=gen) * 0.01).to(torch.bfloat16)
        dyT, dysT = mx.alloc_cols_outputs(sg.M_cap, Ng, Gg, dev)
        mx.mxfp4_bf16_to_fp8_cols_ragged(grad, dyT, dysT, seg0["offs"])
        del grad
        dw = torch.empty((Gg * Ng * Kg,), dtype=torch.int16, device=dev)
        wms = time_launches(lambda: mx.mxfp4_fp8_grouped_gemm_wgrad(
            dyT, dysT, seg0["yT"], seg0["ysT"], dw, seg0["offs"], N=Ng, K=Kg, G=Gg, M_cap=sg.M_cap))
        wgrad = mfma_entry("weight-gradient GEMM: column-quantized [M, N] gradient x hidden-segment FP8 column "
                           "output -> BF16 dW [G, N, K]",
                           {"M_tot": sg.M_tot, "K": Kg, "N": Ng, "G": Gg}, 2.0 * sg.M_tot * Ng * Kg, wms)
        del dyT, dysT, dw

    # the NVFP4 variant quantizer on the forward segments (not in `value`): one call is
    # the amax reset, the tensor amax and the quantizer; its bytes are both reads of x
    # (the per-tensor scale needs the whole tensor first), the codes and the scales
    nvfp4 = []
    for d in segs:
        sg = d["seg"]
        if sg.K % 16:
            continue
        nc, ns, na = mx.alloc_nvfp4_outputs(sg.M_cap, sg.K, dev)
        n_el = sg.M_tot * sg.K
        nbytes = int(n_el * (2 + 2 + 0.5 + 1 / 16))
        # nearest even, then stochastic rounding (Philox4x32-10 bits, a fixed seed)
        for rounding, seed in (("nearest_even", None), ("stochastic", 0x5EED)):
            nms = time_launches(lambda d=d, seed=seed: mx.mxfp4_nvfp4_quantize_rows(d["x"], nc, ns, na, d["offs"],
                                                                                    seed=seed))
            us = float(np.mean(nms)) * 1000.0
            gbs = nbytes / (us * 1e-6) / 1e9
            nvfp4.append({"segment": sg.name, "rounding": rounding, "bytes_per_call": nbytes,
                          "mean_us": round(us, 2), "median_us": round(float(np.median(nms)) * 1000.0, 2),
                          "GBps": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)})
            log(f"[bench] nvfp4 {rounding} {sg.name}: {us:.1f} us per call (3 launches), {gbs:.0f} GB/s "
                f"({gbs / HBM_PEAK_GBS:.1%} of 8 TB/s)")
        del nc, ns, na

    # the backward FP8 quantizer on the same segments, timed the same way (not in `value`)
    bsegs, blaunches = build_launches(mx, w, dev, torch, backward=True)
    for _ in range(args.warmup):
        for _, _, fn, _ in blaunches:
            fn()
    nb_l = len(blaunches)
    bev = KernelEvents(args.steps * nb_l)
    torch.cuda.synchronize()
    tb0 = time.perf_counter()
    for s in range(args.steps):
        for i, (_, _, fn, _) in enumerate(blaunches):
            bev.arm(mx, s * nb_l + i)
            fn()
    torch.cuda.synchronize()
    b_ms_per_step = (time.perf_counter() - tb0) * 1000.0 / args.steps
    bus = bev.elapsed()
    bev.close()
    b_per_kernel = []
    for i, (kern, segname, _, nbytes) in enumerate(blaunches):
        ms = [bus[s * nb_l + i] / 1000.0 for s in range(args.steps)]
        mean_ms = float(np.mean(ms))
        b_per_kernel.append({
            "kernel": kern, "segment": segname, "alg_bytes": nbytes,
            "mean_us": round(mean_ms * 1000.0, 2), "median_us": round(float(np.median(ms)) * 1000.0, 2),
            "GBps": round(nbytes / (mean_ms / 1000.0) / 1e9, 1),
            "frac_of_peak": round(nbytes / (mean_ms / 1000.0) / 1e9 / HBM_PEAK_GBS, 4),
        })
    b_step_bytes = sum(l[3] for l in blaunches)
    backward = {
        "what": "backward FP8 gradient quantizer (BF16 -> E4M3, 1x128 blocks), row and transposed "
                "column layout, per segment",
        "alg_bytes_per_step": b_step_bytes,
        "ms_per_step": round(b_ms_per_step, 4),
        "GBps": round(b_step_bytes / (b_ms_per_step / 1000.0) / 1e9, 1),
        "per_kernel": b_per_kernel,
    }
    # the same quantizer writing both layouts from one read of the gradient
    both = []
    for d in bsegs:
        sg = d["seg"]
        yb, ysb = mx.alloc_fp8q_rows_outputs(sg.M_cap, sg.K, dev)
        yTb, ysTb = mx.alloc_cols_outputs(sg.M_cap, sg.K, sg.G, dev)
        fms = time_launches(lambda d=d: mx.mxfp4_bf16_to_fp8_rows_cols_ragged(d["x"], yb, ysb, yTb, ysTb, d["offs"]))
        nb = (np.diff(sg.offs.astype(np.int64)) + 127) // 128
        nbytes = int(sg.M_tot * sg.K * (2 + 1 + 1 / 128 + 1) + int(nb.sum()) * sg.K)
        us = float(np.mean(fms)) * 1000.0
        gbs = nbytes / (us * 1e-6) / 1e9
        sep = sum(p["mean_us"] for p in b_per_kernel if p["segment"] == sg.name)
        both.append({"segment": sg.name, "alg_bytes": nbytes, "mean_us": round(us, 2),
                     "median_us": round(float(np.median(fms)) * 1000.0, 2), "GBps": round(gbs, 1),
                     "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4), "separate_mean_us": round(sep, 2)})
        log(f"[bench] both layouts {sg.name}: {us:.1f} us ({gbs:.0f} GB/s, {gbs / HBM_PEAK_GBS:.1%} of 8 TB/s) "
            f"against {sep:.1f} us for the two separate launches")
        del yb, ysb, yTb, ysTb
    backward["both_layouts"] = both
    del bsegs, blaunches, bev

    if args.calibrate_copy:
        # three copies of exactly 1 GiB by the hand-written copy kernel (unroll 4), whose
        # HBM counters scale the counters of the kernels above
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty(n, dtype=torch.uint8, device=dev)
        cp = DeviceCopy.__new__(DeviceCopy)
        cp.torch, cp.unroll = torch, 4
        cp.lib = DeviceCopy.load()
        torch.cuda.synchronize()
        for _ in range(3):
            cp(b, a)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy (copy16_kernel<4>): 3 x {n} bytes read + {n} bytes written")
        del a, b

    value = step_bytes / (ms_per_step / 1000.0) / 1e9
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE,
        "data": "synthetic",
        "config": {
            "workload": w.name + ": " + w.description,
            "segments": [{"name": d["seg"].name, "M_cap": d["seg"].M_cap, "M_tot": d["seg"].M_tot,
                          "K": d["seg"].K, "G": d["seg"].G} for d in segs],
            "kernels_per_step": [f"{k}/{s}" for k, s, _, _ in launches],
            "alg_bytes_per_step": step_bytes,
            "frac_of_peak": round(value / HBM_PEAK_GBS, 4),
            "device": props.name,
            "cus": props.multi_processor_count,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": f"{dom['kernel']}/{dom['segment']}",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "alg_bytes_per_launch": dom["alg_bytes"],
            "mean_launch_us": dom["mean_us"],
            "measured": "HIP events bound to this launch's kernel (mxfp4_time_next_launch) inside the timed region",
        },
        "per_kernel": per_kernel,
        "per_kernel_measured": "HIP events bound to every launch's kernel, in an untimed pass of the same steps "
                               "before the timed region",
        "backward": backward,
        "gemm": gemm,
        "wgrad": wgrad,
        "nvfp4": nvfp4,
        "per_config_scrubbed": None,
        "cpu_baseline": None,
    }
    if not args.no_scrubbed:
        del segs, launches
        torch.cuda.empty_cache()
        log("[bench] per-kernel medians with the caches scrubbed (configs 2, 3, 4, 5)")
        result["per_config_scrubbed"] = scrubbed_medians(mx, torch, dev, (2, 3, 4, 5))
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
