"""CPU oracle for the BF16 -> MXFP4 -> block-scaled FP8 path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
(``block_scaled_precision_bf16tofp4row_amd``) never imports it and shares no
code with it.

The arithmetic lives in ``oracle.c`` (plain C, double precision, one element at
a time).  This module compiles it with gcc, loads it with ctypes and splits big
matrices into row ranges that run on a thread pool (ctypes releases the GIL, so
each thread runs the unchanged C code on its own range).

Method: "Practical FP4 Training for Large-Scale MoE Models on Hopper GPUs",
technical summary section 2 "Methodology" (MXFP4 spec, direct FP4->FP8
conversion with hierarchical scale alignment, row / transposed-column kernels
over ragged expert segments).  The conventions the page leaves open are stated
in the header of ``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


def compile_oracle(src: str, out: str) -> str:
    """gcc one oracle source into a shared library (plain -O2, no fast-math)."""
    tmp = out + ".tmp"
    subprocess.check_call(
        ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
         "-ffp-contract=off", "-o", tmp, src, "-lm"])
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so."""
    if force or not os.path.exists(_LIB):
        compile_oracle(_SRC, _LIB)
    return _LIB


# The pins' own test loads deliberately broken copies of oracle.c through this
# variable (one per test process) to show that each plausible mistake fails a pin.
_LIB_OVERRIDE = "MXFP4_ORACLE_LIB"


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get(_LIB_OVERRIDE)
    if not path:
        path = _LIB
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.oracle_quantize_block.argtypes = [P, P, P]
    lib.oracle_quantize_rows.argtypes = [P, I64, I64, I64, P, P]
    lib.oracle_fp8_rows.argtypes = [P, P, I64, I64, I64, P, P]
    lib.oracle_fp8_cols.argtypes = [P, P, P, ctypes.c_int32, I64, I64, I64, P, P]
    lib.oracle_e2m1_encode.argtypes = [ctypes.c_double]
    lib.oracle_e2m1_encode.restype = ctypes.c_int
    lib.oracle_e4m3_encode.argtypes = [ctypes.c_double]
    lib.oracle_e4m3_encode.restype = ctypes.c_int
    lib.oracle_e2m1_magnitude.argtypes = [ctypes.c_int]
    lib.oracle_e2m1_magnitude.restype = ctypes.c_double
    lib.oracle_bf16_value.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_value.restype = ctypes.c_double
    lib.oracle_scale_for_amax.argtypes = [ctypes.c_double]
    lib.oracle_scale_for_amax.restype = ctypes.c_int
    lib.oracle_fp8_of_code.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.oracle_fp8q_block.argtypes = [P, P, P]
    lib.oracle_fp8q_rows.argtypes = [P, I64, I64, I64, P, P]
    lib.oracle_fp8q_cols.argtypes = [P, P, ctypes.c_int32, I64, I64, I64, P, P]
    lib.oracle_fp8_gemm_at.argtypes = [P, P, P, P, P, ctypes.c_int32, I64, I64, P, P, I64, P, P, P]
    lib.oracle_fp8_wgrad_at.argtypes = [P, P, P, P, P, ctypes.c_int32, I64, I64, P, P, P, I64, P, P, P]
    F = ctypes.c_float
    lib.oracle_nvfp4_block.argtypes = [P, F, P, P]
    lib.oracle_nvfp4_amax.argtypes = [P, I64, I64, I64]
    lib.oracle_nvfp4_amax.restype = F
    lib.oracle_nvfp4_encode_scale.argtypes = [F]
    lib.oracle_nvfp4_encode_scale.restype = F
    lib.oracle_nvfp4_rows.argtypes = [P, I64, I64, I64, F, P, P]
    U64 = ctypes.c_uint64
    lib.oracle_philox4x32_10.argtypes = [P, P, P]
    lib.oracle_sr_bits16.argtypes = [U64, I64, I64, I64]
    lib.oracle_sr_bits16.restype = ctypes.c_uint
    lib.oracle_e2m1_encode_sr.argtypes = [ctypes.c_double, ctypes.c_uint]
    lib.oracle_e2m1_encode_sr.restype = ctypes.c_int
    lib.oracle_nvfp4_rows_sr.argtypes = [P, I64, I64, I64, F, U64, P, P]
    lib.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_value.restype = ctypes.c_double
    lib.oracle_bf16_round.argtypes = [ctypes.c_double]
    lib.oracle_bf16_round.restype = ctypes.c_uint16
    lib.oracle_scale_for_amax_e4m3.argtypes = [ctypes.c_double]
    lib.oracle_scale_for_amax_e4m3.restype = ctypes.c_int
    lib.oracle_fp8_of_code.restype = ctypes.c_uint8
    _lib = lib
    return lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def default_threads() -> int:
    """Host threads the multi-range drivers use (the process's CPU affinity)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def _ranges(n: int, parts: int):
    parts = max(1, min(parts, n)) if n > 0 else 1
    step = (n + parts - 1) // parts if n > 0 else 0
    return [(i, min(n, i + step)) for i in range(0, n, step)] if n > 0 else []


# ---- scalar helpers (used by the pins) -------------------------------------

def e2m1_encode(y: float) -> int:
    return _load().oracle_e2m1_encode(float(y))


def e4m3_encode(v: float) -> int:
    return _load().oracle_e4m3_encode(float(v))


def e2m1_magnitude(code: int) -> float:
    return _load().oracle_e2m1_magnitude(int(code))


def bf16_value(bits: int) -> float:
    return _load().oracle_bf16_value(int(bits))


def scale_for_amax(amax: float) -> int:
    return _load().oracle_scale_for_amax(float(amax))


def fp8_of_code(code: int, s: int, S: int) -> int:
    return _load().oracle_fp8_of_code(int(code), int(s), int(S))


# ---- array drivers -----------------------------------------------------------

def quantize_block(x32: np.ndarray):
    """One 32-element block of BF16 bits -> (16 packed bytes, scale byte)."""
    lib = _load()
    x32 = np.ascontiguousarray(x32, dtype=np.uint16)
    assert x32.size == 32
    packed = np.zeros(16, np.uint8)
    sc = np.zeros(1, np.uint8)
    lib.oracle_quantize_block(_ptr(x32), _ptr(packed), _ptr(sc))
    return packed, int(sc[0])


def quantize_rows(x_bits: np.ndarray, rows: int | None = None, threads: int = 1,
                  codes: np.ndarray | None = None, scales: np.ndarray | None = None):
    """BF16 bits [M, K] -> (codes [M, K/2] uint8, scales [M, K/32] uint8).

    Only rows [0, rows) are computed (rows defaults to M); the rest stay zero."""
    lib = _load()
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    M, K = x_bits.shape
    assert K % 32 == 0
    rows = M if rows is None else rows
    if codes is None:
        codes = np.zeros((M, K // 2), np.uint8)
    if scales is None:
        scales = np.zeros((M, K // 32), np.uint8)

    def run(r):
        lib.oracle_quantize_rows(_ptr(x_bits), K, r[0], r[1], _ptr(codes), _ptr(scales))

    _run_ranges(run, _ranges(rows, threads * 4), threads)
    return codes, scales


def nvfp4_block(x16_bits, t: float):
    """One 16-element NVFP4 block with the tensor's FP32 encode scale t:
    (8 packed code bytes, E4M3 scale byte)."""
    lib = _load()
    x = np.ascontiguousarray(x16_bits, dtype=np.uint16)
    assert x.size == 16
    packed = np.zeros(8, np.uint8)
    sc = np.zeros(1, np.uint8)
    lib.oracle_nvfp4_block(_ptr(x), float(t), _ptr(packed), _ptr(sc))
    return packed, int(sc[0])


def nvfp4_encode_scale(amax: float) -> float:
    """FP32(2688 / amax) (1 for 0, FLT_MAX on overflow), as an FP32 value."""
    return float(_load().oracle_nvfp4_encode_scale(float(amax)))


def nvfp4_quantize_rows(x_bits: np.ndarray, rows: int | None = None, threads: int = 1):
    """NVFP4 over rows [0, rows) of BF16 bits [M, K] (K a multiple of 16):
    (codes [M, K/2], E4M3 block scales [M, K/16], tensor amax, FP32 encode scale t);
    rows past `rows` stay zero."""
    lib = _load()
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    M, K = x_bits.shape
    assert K % 16 == 0
    rows = M if rows is None else rows
    codes = np.zeros((M, K // 2), np.uint8)
    scales = np.zeros((M, K // 16), np.uint8)
    parts = []

    def run_amax(r):
        parts.append(float(lib.oracle_nvfp4_amax(_ptr(x_bits), K, r[0], r[1])))

    _run_ranges(run_amax, _ranges(rows, threads * 4), threads)
    amax = max(parts) if parts else 0.0
    t = nvfp4_encode_scale(amax)

    def run(r):
        lib.oracle_nvfp4_rows(_ptr(x_bits), K, r[0], r[1], t, _ptr(codes), _ptr(scales))

    _run_ranges(run, _ranges(rows, threads * 4), threads)
    return codes, scales, amax, t


def philox4x32_10(counter, key) -> list[int]:
    """Philox4x32-10 (Salmon et al., SC'11): four 32-bit counter words and two key
    words -> four output words."""
    lib = _load()
    c = np.ascontiguousarray(counter, np.uint32)
    k = np.ascontiguousarray(key, np.uint32)
    out = np.zeros(4, np.uint32)
    lib.oracle_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return [int(v) for v in out]


def sr_bits16(seed: int, K: int, m: int, k: int) -> int:
    """The 16 random bits that element (m, k) of a [*, K] matrix draws under `seed`."""
    return int(_load().oracle_sr_bits16(seed, K, m, k))


def e2m1_encode_sr(a: float, r: int) -> int:
    """E2M1 magnitude code of a >= 0 rounded stochastically with the 16-bit random r."""
    return int(_load().oracle_e2m1_encode_sr(a, r))


def nvfp4_quantize_rows_sr(x_bits: np.ndarray, seed: int, rows: int | None = None, threads: int = 1):
    """NVFP4 as nvfp4_quantize_rows with the element codes rounded stochastically
    (Philox4x32-10 random bits under `seed`); block scales, amax and t unchanged."""
    lib = _load()
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    M, K = x_bits.shape
    assert K % 16 == 0
    rows = M if rows is None else rows
    codes = np.zeros((M, K // 2), np.uint8)
    scales = np.zeros((M, K // 16), np.uint8)
    parts = []

    def run_amax(r):
        parts.append(float(lib.oracle_nvfp4_amax(_ptr(x_bits), K, r[0], r[1])))

    _run_ranges(run_amax, _ranges(rows, threads * 4), threads)
    amax = max(parts) if parts else 0.0
    t = nvfp4_encode_scale(amax)

    def run(r):
        lib.oracle_nvfp4_rows_sr(_ptr(x_bits), K, r[0], r[1], t, seed, _ptr(codes), _ptr(scales))

    _run_ranges(run, _ranges(rows, threads * 4), threads)
    return codes, scales, amax, t


def fp8_rows(codes: np.ndarray, scales: np.ndarray, rows: int | None = None,
             threads: int = 1, y: np.ndarray | None = None, y_scales: np.ndarray | None = None):
    """Row layout: codes [M, K/2], scales [M, K/32] -> (y [M, K], y_scales [M, K/128])."""
    lib = _load()
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    M = codes.shape[0]
    K = codes.shape[1] * 2
    assert K % 128 == 0 and scales.shape == (M, K // 32)
    rows = M if rows is None else rows
    if y is None:
        y = np.zeros((M, K), np.uint8)
    if y_scales is None:
        y_scales = np.zeros((M, K // 128), np.uint8)

    def run(r):
        lib.oracle_fp8_rows(_ptr(codes), _ptr(scales), K, r[0], r[1], _ptr(y), _ptr(y_scales))

    _run_ranges(run, _ranges(rows, threads * 4), threads)
    return y, y_scales


def scale_for_amax_e4m3(amax: float) -> int:
    return _load().oracle_scale_for_amax_e4m3(float(amax))


def fp8q_block(x128: np.ndarray):
    """One 128-element block of BF16 bits -> (128 E4M3 bytes, UE8M0 scale byte)."""
    lib = _load()
    x128 = np.ascontiguousarray(x128, dtype=np.uint16)
    assert x128.size == 128
    y = np.zeros(128, np.uint8)
    sc = np.zeros(1, np.uint8)
    lib.oracle_fp8q_block(_ptr(x128), _ptr(y), _ptr(sc))
    return y, int(sc[0])


def fp8q_rows(x_bits: np.ndarray, rows: int | None = None, threads: int = 1,
              y: np.ndarray | None = None, y_scales: np.ndarray | None = None):
    """Backward FP8 quantizer, row layout: BF16 bits [M, K] -> (y [M, K] E4M3 bytes,
    y_scales [M, K/128] UE8M0 bytes).  Only rows [0, rows) are computed."""
    lib = _load()
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    M, K = x_bits.shape
    assert K % 128 == 0
    rows = M if rows is None else rows
    if y is None:
        y = np.zeros((M, K), np.uint8)
    if y_scales is None:
        y_scales = np.zeros((M, K // 128), np.uint8)

    def run(r):
        lib.oracle_fp8q_rows(_ptr(x_bits), K, r[0], r[1], _ptr(y), _ptr(y_scales))

    _run_ranges(run, _ranges(rows, threads * 4), threads)
    return y, y_scales


def blocks_per_group(offs: np.ndarray) -> np.ndarray:
    counts = np.diff(np.asarray(offs, dtype=np.int64))
    return (counts + 127) // 128


def cols_scale_size(offs: np.ndarray, K: int) -> int:
    return int(blocks_per_group(offs).sum()) * K


def fp8_cols(codes: np.ndarray, scales: np.ndarray, offs: np.ndarray, threads: int = 1,
             yT: np.ndarray | None = None, yT_scales: np.ndarray | None = None,
             groups=None):
    """Transposed column layout over ragged expert segments.

    Returns (yT, yT_scales) as flat uint8 arrays: expert g's [K, M_g] transpose
    at byte K*offs[g], its [nblocks_g, K] scales at byte K*B_g."""
    lib = _load()
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    offs = np.ascontiguousarray(offs, dtype=np.int32)
    M = codes.shape[0]
    K = codes.shape[1] * 2
    G = offs.size - 1
    assert K % 128 == 0
    if yT is None:
        yT = np.zeros(M * K, np.uint8)
    if yT_scales is None:
        yT_scales = np.zeros(max(1, cols_scale_size(offs, K)), np.uint8)
    nbg = blocks_per_group(offs)
    groups = range(G) if groups is None else groups
    work = []
    for g in groups:
        for b0, b1 in _ranges(int(nbg[g]), max(1, threads)):
            work.append((g, b0, b1))

    def run(w):
        lib.oracle_fp8_cols(_ptr(codes), _ptr(scales), _ptr(offs), w[0], K, w[1], w[2],
                            _ptr(yT), _ptr(yT_scales))

    _run_ranges(run, work, threads)
    return yT, yT_scales


def _run_ranges(fn, work, threads):
    if threads <= 1 or len(work) <= 1:
        for w in work:
            fn(w)
        return
    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(fn, work))


def fp8q_cols(x_bits: np.ndarray, offs: np.ndarray, threads: int = 1,
              yT: np.ndarray | None = None, yT_scales: np.ndarray | None = None, groups=None):
    """Backward FP8 quantizer, transposed column layout over ragged expert segments:
    BF16 bits [M, K] -> flat (yT, yT_scales), expert g's [K, M_g] transpose at byte
    K*offs[g] and its [nblocks_g, K] scales at byte K*B_g (the layout of fp8_cols)."""
    lib = _load()
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    offs = np.ascontiguousarray(offs, dtype=np.int32)
    M, K = x_bits.shape
    G = offs.size - 1
    assert K % 128 == 0
    if yT is None:
        yT = np.zeros(M * K, np.uint8)
    if yT_scales is None:
        yT_scales = np.zeros(max(1, cols_scale_size(offs, K)), np.uint8)
    nbg = blocks_per_group(offs)
    groups = range(G) if groups is None else groups
    work = []
    for g in groups:
        for b0, b1 in _ranges(int(nbg[g]), max(1, threads)):
            work.append((g, b0, b1))

    def run(w):
        lib.oracle_fp8q_cols(_ptr(x_bits), _ptr(offs), w[0], K, w[1], w[2], _ptr(yT), _ptr(yT_scales))

    _run_ranges(run, work, threads)
    return yT, yT_scales


# ---- FP8 grouped GEMM (forward, row layout) -----------------------------------------

def e4m3_value(b: int) -> float:
    return _load().oracle_e4m3_value(int(b))


def bf16_round(v: float) -> int:
    return int(_load().oracle_bf16_round(float(v)))


def fp8_gemm_at(a, sa, w, sw, offs, ms, ns, threads: int = 1):
    """The expert-grouped FP8 GEMM at the points (ms[i], ns[i]).

    a [M, K] E4M3 bytes, sa [M, K/128] UE8M0, w [G, N, K] E4M3, sw [G, N, K/128] UE8M0,
    offs [G+1] int32.  Returns (exact fp64 values, BF16 bits, sum of |terms|)."""
    lib = _load()
    a = np.ascontiguousarray(a, dtype=np.uint8)
    sa = np.ascontiguousarray(sa, dtype=np.uint8)
    w = np.ascontiguousarray(w, dtype=np.uint8)
    sw = np.ascontiguousarray(sw, dtype=np.uint8)
    offs = np.ascontiguousarray(offs, dtype=np.int32)
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    G, N, K = w.shape
    assert K % 128 == 0 and a.shape[1] == K and ms.shape == ns.shape
    cnt = ms.size
    exact = np.zeros(cnt, np.float64)
    ybf = np.zeros(cnt, np.uint16)
    absum = np.zeros(cnt, np.float64)

    def run(r):
        lo, hi = r
        lib.oracle_fp8_gemm_at(_ptr(a), _ptr(sa), _ptr(w), _ptr(sw), _ptr(offs), G, N, K,
                               _ptr(ms[lo:]), _ptr(ns[lo:]), hi - lo,
                               _ptr(exact[lo:]), _ptr(ybf[lo:]), _ptr(absum[lo:]))

    _run_ranges(run, _ranges(cnt, threads * 4), threads)
    return exact, ybf, absum


def fp8_wgrad_at(dyT, dyT_scales, xT, xT_scales, offs, N, K, gs, ns, ks, threads: int = 1):
    """The weight-gradient GEMM over the column layouts at the points (gs[i], ns[i], ks[i]):
    dW[g, n, k] = sum over expert g's tokens of dY_g[m, n] X_g[m, k].  dyT / xT are the
    column-layout outputs for widths N / K (oracle.fp8q_cols / oracle.fp8_cols).
    Returns (exact fp64 values, BF16 bits, sum of |terms|)."""
    lib = _load()
    dyT = np.ascontiguousarray(dyT, dtype=np.uint8)
    dyT_scales = np.ascontiguousarray(dyT_scales, dtype=np.uint8)
    xT = np.ascontiguousarray(xT, dtype=np.uint8)
    xT_scales = np.ascontiguousarray(xT_scales, dtype=np.uint8)
    offs = np.ascontiguousarray(offs, dtype=np.int32)
    gs = np.ascontiguousarray(gs, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    ks = np.ascontiguousarray(ks, dtype=np.int64)
    G = offs.size - 1
    assert gs.shape == ns.shape == ks.shape
    assert dyT.size >= N * int(offs[-1]) and xT.size >= K * int(offs[-1])
    assert dyT_scales.size >= cols_scale_size(offs, N) and xT_scales.size >= cols_scale_size(offs, K)
    assert np.all((gs >= 0) & (gs < G) & (ns >= 0) & (ns < N) & (ks >= 0) & (ks < K))
    cnt = gs.size
    exact = np.zeros(cnt, np.float64)
    ybf = np.zeros(cnt, np.uint16)
    absum = np.zeros(cnt, np.float64)

    def run(r):
        lo, hi = r
        lib.oracle_fp8_wgrad_at(_ptr(dyT), _ptr(dyT_scales), _ptr(xT), _ptr(xT_scales), _ptr(offs), G, N, K,
                                _ptr(gs[lo:]), _ptr(ns[lo:]), _ptr(ks[lo:]), hi - lo,
                                _ptr(exact[lo:]), _ptr(ybf[lo:]), _ptr(absum[lo:]))

    _run_ranges(run, _ranges(cnt, threads * 4), threads)
    return exact, ybf, absum


def fp8_wgrad(dyT, dyT_scales, xT, xT_scales, offs, N, K, threads: int = 1):
    """Every output of the weight-gradient GEMM: (exact [G, N, K] fp64, BF16 bits, absum)."""
    G = np.asarray(offs).size - 1
    gg, nn, kk = np.meshgrid(np.arange(G, dtype=np.int64), np.arange(N, dtype=np.int64),
                             np.arange(K, dtype=np.int64), indexing="ij")
    e, y, t = fp8_wgrad_at(dyT, dyT_scales, xT, xT_scales, offs, N, K, gg.reshape(-1), nn.reshape(-1),
                           kk.reshape(-1), threads)
    return e.reshape(G, N, K), y.reshape(G, N, K), t.reshape(G, N, K)


def fp8_gemm(a, sa, w, sw, offs, threads: int = 1):
    """Every output of the GEMM: (exact [M_tot, N] fp64, BF16 bits [M_tot, N], absum)."""
    G, N, K = np.asarray(w).shape
    M_tot = int(np.asarray(offs)[-1])
    mm, nn = np.meshgrid(np.arange(M_tot, dtype=np.int64), np.arange(N, dtype=np.int64), indexing="ij")
    e, y, t = fp8_gemm_at(a, sa, w, sw, offs, mm.reshape(-1), nn.reshape(-1), threads)
    return e.reshape(M_tot, N), y.reshape(M_tot, N), t.reshape(M_tot, N)
