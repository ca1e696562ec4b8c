"""Helpers for the GPU parity tests: run the HIP path through the C ABI (via the
thin binding) on one segment, run the oracle on the same bytes, compare byte by
byte, and check that every byte outside the documented output ranges keeps its
canary value."""
from __future__ import annotations

import numpy as np
import torch

import block_scaled_precision_bf16tofp4row_amd as mx
import oracle

CANARY = 0xA5


def dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy()


def canary(shape) -> torch.Tensor:
    return torch.full(shape, CANARY, dtype=torch.uint8, device="cuda")


def gpu_quantize(x_bits: np.ndarray, offs: np.ndarray, x_d=None, offs_d=None):
    M_cap, K = x_bits.shape
    x_d = dev(x_bits) if x_d is None else x_d
    offs_d = dev(offs) if offs_d is None else offs_d
    codes = canary((M_cap, K // 2))
    scales = canary((M_cap, K // 32))
    mx.mxfp4_quantize_rows(x_d, codes, scales, offs_d)
    return codes, scales


def gpu_rows(codes_d, scales_d, offs_d, M_cap, K):
    y = canary((M_cap, K))
    ys = canary((M_cap, K // 128))
    mx.mxfp4_to_fp8_rows(codes_d, scales_d, y, ys, offs_d, M_cap=M_cap, K=K)
    return y, ys


def gpu_cols(codes_d, scales_d, offs_d, M_cap, K, G):
    yT = canary((max(1, M_cap * K),))
    cap = mx.mxfp4_cols_scale_capacity(M_cap, K, G)
    ys = canary((max(1, cap),))
    mx.mxfp4_to_fp8_cols_ragged(codes_d, scales_d, yT, ys, offs_d, G=G, M_cap=M_cap, K=K)
    return yT, ys


def gpu_fp8q_rows(x_d, offs_d, M_cap, K):
    y = canary((M_cap, K))
    ys = canary((M_cap, K // 128))
    mx.mxfp4_bf16_to_fp8_rows(x_d, y, ys, offs_d, M_cap=M_cap, K=K)
    return y, ys


def check_fp8q_rows(x_bits: np.ndarray, offs: np.ndarray, threads: int | None = None):
    """Backward FP8 quantizer, row layout: GPU vs oracle on rows [0, offs[G]), canary
    beyond."""
    threads = oracle.default_threads() if threads is None else threads
    M_cap, K = x_bits.shape
    M_tot = int(offs[-1])
    y_d, ys_d = gpu_fp8q_rows(dev(x_bits), dev(offs), M_cap, K)
    y_o, ys_o = oracle.fp8q_rows(x_bits, rows=M_tot, threads=threads)
    y_g, ys_g = host(y_d), host(ys_d)
    assert_bytes_equal(ys_g[:M_tot], ys_o[:M_tot], "fp8q row scales", row_len=K // 128)
    assert_bytes_equal(y_g[:M_tot], y_o[:M_tot], "fp8q rows", row_len=K)
    assert_untouched(y_g[M_tot:], "fp8q rows past offs[G]")
    assert_untouched(ys_g[M_tot:], "fp8q row scales past offs[G]")


def gpu_fp8q_cols(x_d, offs_d, M_cap, K, G):
    yT = canary((max(1, M_cap * K),))
    cap = mx.mxfp4_cols_scale_capacity(M_cap, K, G)
    ys = canary((max(1, cap),))
    mx.mxfp4_bf16_to_fp8_cols_ragged(x_d, yT, ys, offs_d, G=G, M_cap=M_cap, K=K)
    return yT, ys


def check_fp8q_cols(x_bits: np.ndarray, offs: np.ndarray, threads: int | None = None):
    """Backward FP8 quantizer, transposed column layout: GPU vs oracle on every expert's
    transpose and scales, canary beyond."""
    threads = oracle.default_threads() if threads is None else threads
    M_cap, K = x_bits.shape
    G = offs.size - 1
    M_tot = int(offs[-1])
    yT_d, ys_d = gpu_fp8q_cols(dev(x_bits), dev(offs), M_cap, K, G)
    used_s = oracle.cols_scale_size(offs, K)
    yT_o = np.full(max(1, M_cap * K), CANARY, np.uint8)
    ys_o = np.full(max(1, used_s), CANARY, np.uint8)
    oracle.fp8q_cols(x_bits, offs, threads=threads, yT=yT_o, yT_scales=ys_o)
    yT_g, ys_g = host(yT_d), host(ys_d)
    assert_bytes_equal(ys_g[:used_s], ys_o[:used_s], "fp8q col scales")
    assert_bytes_equal(yT_g[:M_tot * K], yT_o[:M_tot * K], "fp8q cols")
    assert_untouched(yT_g[M_tot * K:], "fp8q cols past K*offs[G]")
    assert_untouched(ys_g[used_s:], "fp8q col scales past the used blocks")


def assert_bytes_equal(got: np.ndarray, want: np.ndarray, what: str, row_len: int | None = None):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if np.array_equal(got, want):
        return
    bad = np.nonzero(got.reshape(-1) != want.reshape(-1))[0]
    lines = []
    for i in bad[:10]:
        loc = (int(i) // row_len, int(i) % row_len) if row_len else int(i)
        lines.append(f"  at {loc}: got 0x{int(got.reshape(-1)[i]):02x} want 0x{int(want.reshape(-1)[i]):02x}")
    raise AssertionError(f"{what}: {bad.size} of {got.size} bytes differ\n" + "\n".join(lines))


def assert_untouched(arr: np.ndarray, what: str):
    arr = np.asarray(arr)
    if arr.size and not np.all(arr == CANARY):
        n = int(np.count_nonzero(arr != CANARY))
        raise AssertionError(f"{what}: {n} bytes outside the output range were written")


def check_chain(x_bits: np.ndarray, offs: np.ndarray, kernels=("quantize", "rows", "cols"),
                threads: int | None = None):
    """Run quantize (+ rows, + cols) on the GPU and compare everything with the oracle."""
    threads = oracle.default_threads() if threads is None else threads
    M_cap, K = x_bits.shape
    G = offs.size - 1
    M_tot = int(offs[-1])
    offs_d = dev(offs)
    codes_d, scales_d = gpu_quantize(x_bits, offs, offs_d=offs_d)
    c_o, s_o = oracle.quantize_rows(x_bits, rows=M_tot, threads=threads)
    c_g, s_g = host(codes_d), host(scales_d)
    assert_bytes_equal(c_g[:M_tot], c_o[:M_tot], "codes", row_len=K // 2)
    assert_bytes_equal(s_g[:M_tot], s_o[:M_tot], "scales", row_len=K // 32)
    assert_untouched(c_g[M_tot:], "codes past offs[G]")
    assert_untouched(s_g[M_tot:], "scales past offs[G]")
    out = {"codes": c_g, "scales": s_g}
    if "rows" in kernels:
        y_d, ys_d = gpu_rows(codes_d, scales_d, offs_d, M_cap, K)
        y_o, ys_o = oracle.fp8_rows(c_o, s_o, rows=M_tot, threads=threads)
        y_g, ysg = host(y_d), host(ys_d)
        assert_bytes_equal(y_g[:M_tot], y_o[:M_tot], "fp8 rows", row_len=K)
        assert_bytes_equal(ysg[:M_tot], ys_o[:M_tot], "fp8 row scales", row_len=K // 128)
        assert_untouched(y_g[M_tot:], "fp8 rows past offs[G]")
        assert_untouched(ysg[M_tot:], "fp8 row scales past offs[G]")
        del y_d, ys_d, y_g, y_o
    if "cols" in kernels:
        yT_d, ysT_d = gpu_cols(codes_d, scales_d, offs_d, M_cap, K, G)
        used_s = oracle.cols_scale_size(offs, K)
        yT_o = np.full(max(1, M_cap * K), CANARY, np.uint8)
        ysT_o = np.full(max(1, used_s), CANARY, np.uint8)
        oracle.fp8_cols(c_o, s_o, offs, threads=threads, yT=yT_o, yT_scales=ysT_o)
        yT_g, ysT_g = host(yT_d), host(ysT_d)
        assert_bytes_equal(yT_g[:M_tot * K], yT_o[:M_tot * K], "fp8 cols")
        assert_untouched(yT_g[M_tot * K:], "fp8 cols past K*offs[G]")
        assert_bytes_equal(ysT_g[:used_s], ysT_o[:used_s], "fp8 col scales")
        assert_untouched(ysT_g[used_s:], "fp8 col scales past the used blocks")
    return out


def check_fp8q_both(x_bits: np.ndarray, offs: np.ndarray, threads: int | None = None):
    """Backward FP8 quantizer, both layouts from one read: the row outputs against the
    oracle's row quantizer and the column outputs against its column quantizer, canary
    beyond both."""
    threads = oracle.default_threads() if threads is None else threads
    M_cap, K = x_bits.shape
    G = offs.size - 1
    M_tot = int(offs[-1])
    y = canary((max(1, M_cap), K))
    ys = canary((max(1, M_cap), K // 128))
    yT = canary((max(1, M_cap * K),))
    cap = mx.mxfp4_cols_scale_capacity(M_cap, K, G)
    ysT = canary((max(1, cap),))
    x_d = dev(x_bits) if M_cap else canary((1, K)).view(torch.int16)
    mx.mxfp4_bf16_to_fp8_rows_cols_ragged(x_d, y, ys, yT, ysT, dev(offs), G=G, M_cap=M_cap, K=K)
    y_o, ys_o = oracle.fp8q_rows(x_bits, rows=M_tot, threads=threads)
    used_s = oracle.cols_scale_size(offs, K)
    yT_o = np.full(max(1, M_cap * K), CANARY, np.uint8)
    ysT_o = np.full(max(1, used_s), CANARY, np.uint8)
    oracle.fp8q_cols(x_bits, offs, threads=threads, yT=yT_o, yT_scales=ysT_o)
    y_g, ys_g, yT_g, ysT_g = host(y), host(ys), host(yT), host(ysT)
    assert_bytes_equal(ys_g[:M_tot], ys_o[:M_tot], "both: row scales", row_len=K // 128)
    assert_bytes_equal(y_g[:M_tot], y_o[:M_tot], "both: rows", row_len=K)
    assert_untouched(y_g[M_tot:], "both: rows past offs[G]")
    assert_untouched(ys_g[M_tot:], "both: row scales past offs[G]")
    assert_bytes_equal(ysT_g[:used_s], ysT_o[:used_s], "both: col scales")
    assert_bytes_equal(yT_g[:M_tot * K], yT_o[:M_tot * K], "both: cols")
    assert_untouched(yT_g[M_tot * K:], "both: cols past K*offs[G]")
    assert_untouched(ysT_g[used_s:], "both: col scales past the used blocks")
