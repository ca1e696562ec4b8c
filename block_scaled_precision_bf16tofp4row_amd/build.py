"""Build libmxfp4cvt.so in-tree with hipcc for gfx950.

    python -m block_scaled_precision_bf16tofp4row_amd.build

Compiles every ``csrc/*.hip`` to an object (in parallel) and links them into
``block_scaled_precision_bf16tofp4row_amd/libmxfp4cvt.so``; then builds the
benchmark's measurement kernels (``csrc/bench/*.hip``: the streaming copy and the
memory-only column traffic) into ``libmxfp4bench.so``, a separate library the product
never loads.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmxfp4cvt.so")
BENCH_SRCS = sorted(glob.glob(os.path.join(CSRC, "bench", "*.hip")))
BENCH_LIB = os.path.join(PKG, "libmxfp4bench.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-I", INCLUDE, "-I", CSRC,
    # packed-FP32 VALU forms stay off: ordinary scalar code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    procs = []
    objs = []
    bench_tmp = BENCH_LIB + ".tmp"
    bench_cmd = [HIPCC, *CFLAGS, "-shared", *BENCH_SRCS, "-o", bench_tmp]
    procs.append(("csrc/bench", subprocess.Popen(bench_cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    for src in sources():
        obj = os.path.join(OBJDIR, os.path.basename(src)[:-4] + ".o")
        objs.append(obj)
        cmd = [HIPCC, *CFLAGS, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # the host pass does not know the device-only feature flag; that note is harmless
        lines = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln]
        if p.returncode != 0:
            failed.append(src)
            print("\n".join(lines), file=sys.stderr)
        elif verbose and lines:
            print("\n".join(lines))
    if failed:
        raise RuntimeError("hipcc failed for: " + ", ".join(failed))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    os.replace(bench_tmp, BENCH_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
