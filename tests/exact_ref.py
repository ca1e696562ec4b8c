"""Brute-force exact reference in rational arithmetic, for tiny inputs.

This is the pin the C oracle is checked against.  It computes every result by
exhaustive nearest-value search over the representable values of each format,
using ``fractions.Fraction`` (exact), and never calls the oracle.

* E2M1 magnitudes come from the bit split (1 sign, 2 exponent, 1 mantissa bit)
  named in "Practical FP4 Training for Large-Scale MoE Models on Hopper GPUs",
  technical summary section 2, item 1; their extreme values are cross-checked
  against the OCP MX v1.0 facts stored in ``tests/golden/formats.json``.
* E4M3 values come from torch's ``float8_e4m3fn`` decoder (a library routine).
* Rounding: nearest value, ties to the code with an even mantissa LSB; E2M1
  saturates at 6 (OCP MX conversion rule).
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction

import numpy as np


def bf16_to_fraction(bits: int) -> Fraction:
    f = struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]
    assert math.isfinite(f)
    return Fraction(f)


def e2m1_code_values() -> list[Fraction]:
    """Magnitudes of codes 0..7 from the bit split: exponent field (2 bits,
    bias 2**(2-1)-1 = 1) and one mantissa bit; exponent field 0 is subnormal."""
    bias = 1
    vals = []
    for code in range(8):
        e, m = code >> 1, code & 1
        if e == 0:
            vals.append(Fraction(m, 2) * Fraction(2) ** (1 - bias))
        else:
            vals.append((1 + Fraction(m, 2)) * Fraction(2) ** (e - bias))
    return vals


_E2M1 = e2m1_code_values()


def e4m3_code_values() -> list[Fraction]:
    """Magnitudes of E4M3FN codes 0x00..0x7E, decoded by torch."""
    import torch
    f = torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float32)
    return [Fraction(float(v)) for v in f.tolist()]


_E4M3 = None


def _e4m3():
    global _E4M3
    if _E4M3 is None:
        _E4M3 = e4m3_code_values()
    return _E4M3


def nearest_even(y: Fraction, values: list[Fraction]) -> int:
    """Index of the value nearest to y; on a tie, the even index."""
    best, bestd = None, None
    for i, v in enumerate(values):
        d = abs(y - v)
        if bestd is None or d < bestd or (d == bestd and i % 2 == 0 and best % 2 == 1):
            best, bestd = i, d
    return best


def e2m1_encode(y: Fraction) -> int:
    if y > _E2M1[-1]:
        return 7  # saturate
    return nearest_even(y, _E2M1)


def e4m3_encode(v: Fraction) -> int:
    vals = _e4m3()
    assert v <= vals[-1]
    return nearest_even(v, vals)


def floor_log2(a: Fraction) -> int:
    e = 0
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def scale_of_block(xs: list[Fraction]) -> int:
    amax = max(abs(v) for v in xs)
    if amax == 0:
        return 0
    return min(254, max(0, floor_log2(amax) - 2 + 127))


def quantize(x_bits: np.ndarray):
    """[M, K] BF16 bits -> (codes [M, K/2], scales [M, K/32])."""
    M, K = x_bits.shape
    codes = np.zeros((M, K // 2), np.uint8)
    scales = np.zeros((M, K // 32), np.uint8)
    for m in range(M):
        for j in range(K // 32):
            bits = [int(b) for b in x_bits[m, 32 * j:32 * j + 32]]
            xs = [bf16_to_fraction(b) for b in bits]
            s = scale_of_block(xs)
            scales[m, j] = s
            for i in range(32):
                y = abs(xs[i]) / Fraction(2) ** (s - 127)
                c = e2m1_encode(y) | (8 if bits[i] & 0x8000 else 0)
                k = 32 * j + i
                if k % 2 == 0:
                    codes[m, k // 2] |= c
                else:
                    codes[m, k // 2] |= c << 4
    return codes, scales


def _code(codes, m, k):
    b = int(codes[m, k // 2])
    return (b >> 4) if k % 2 else (b & 15)


def _fp8(c: int, s: int, S: int) -> int:
    v = _E2M1[c & 7] * Fraction(2) ** (s - S)
    return e4m3_encode(v) | (0x80 if c & 8 else 0)


def fp8_rows(codes: np.ndarray, scales: np.ndarray):
    M = codes.shape[0]
    K = codes.shape[1] * 2
    y = np.zeros((M, K), np.uint8)
    ys = np.zeros((M, K // 128), np.uint8)
    for m in range(M):
        for b in range(K // 128):
            S = max(int(scales[m, 4 * b + j]) for j in range(4))
            ys[m, b] = S
            for k in range(128 * b, 128 * b + 128):
                y[m, k] = _fp8(_code(codes, m, k), int(scales[m, k // 32]), S)
    return y, ys


def fp8_cols(codes: np.ndarray, scales: np.ndarray, offs: np.ndarray):
    """Per expert g: transpose [K, M_g] at K*offs[g]; scales [nb_g, K] at K*B_g."""
    K = codes.shape[1] * 2
    M = codes.shape[0]
    G = len(offs) - 1
    nb = [(int(offs[g + 1]) - int(offs[g]) + 127) // 128 for g in range(G)]
    yT = np.zeros(M * K, np.uint8)
    ys = np.zeros(max(1, sum(nb) * K), np.uint8)
    B = 0
    for g in range(G):
        r0 = int(offs[g])
        Mg = int(offs[g + 1]) - r0
        for b in range(nb[g]):
            rows = range(r0 + 128 * b, r0 + min(Mg, 128 * b + 128))
            for k in range(K):
                j = k // 32
                S = max(int(scales[m, j]) for m in rows)
                ys[K * (B + b) + k] = S
                for m in rows:
                    yT[K * r0 + k * Mg + (m - r0)] = _fp8(_code(codes, m, k), int(scales[m, j]), S)
        B += nb[g]
    return yT, ys


# ---- backward FP8 quantizer: BF16 -> E4M3 with 1x128 blocks along the row -----------
# Scale: the OCP MX rule with E4M3's largest exponent, floor(log2 amax) - 8 + 127,
# clamped to [0, 254], 0 for an all-zero block.  Elements: nearest E4M3FN value of
# |x| / 2^(S-127), ties to the even code, values above the largest finite value (448)
# clamped to it (the OCP MX conversion rule for FP8 targets), sign kept.

def e4m3_encode_saturating(v: Fraction) -> int:
    vals = _e4m3()
    if v > vals[-1]:
        return len(vals) - 1
    return nearest_even(v, vals)


def scale_of_block_e4m3(xs: list[Fraction]) -> int:
    amax = max(abs(v) for v in xs)
    if amax == 0:
        return 0
    return min(254, max(0, floor_log2(amax) - 8 + 127))


def fp8q_rows(x_bits: np.ndarray):
    """[M, K] BF16 bits -> (y [M, K] E4M3 bytes, y_scales [M, K/128])."""
    M, K = x_bits.shape
    y = np.zeros((M, K), np.uint8)
    ys = np.zeros((M, K // 128), np.uint8)
    for m in range(M):
        for b in range(K // 128):
            bits = [int(v) for v in x_bits[m, 128 * b:128 * b + 128]]
            xs = [bf16_to_fraction(v) for v in bits]
            S = scale_of_block_e4m3(xs)
            ys[m, b] = S
            for i in range(128):
                v = abs(xs[i]) / Fraction(2) ** (S - 127)
                y[m, 128 * b + i] = e4m3_encode_saturating(v) | (0x80 if bits[i] & 0x8000 else 0)
    return y, ys


def fp8q_cols(x_bits: np.ndarray, offs: np.ndarray):
    """Per expert g: E4M3 transpose [K, M_g] at K*offs[g]; scales [nb_g, K] at K*B_g;
    the 1x128 blocks run along the token dimension of each expert."""
    M, K = x_bits.shape
    G = len(offs) - 1
    nb = [(int(offs[g + 1]) - int(offs[g]) + 127) // 128 for g in range(G)]
    yT = np.zeros(M * K, np.uint8)
    ys = np.zeros(max(1, sum(nb) * K), np.uint8)
    B = 0
    for g in range(G):
        r0 = int(offs[g])
        Mg = int(offs[g + 1]) - r0
        for b in range(nb[g]):
            rows = range(r0 + 128 * b, r0 + min(Mg, 128 * b + 128))
            for k in range(K):
                xs = [bf16_to_fraction(int(x_bits[m, k])) for m in rows]
                S = scale_of_block_e4m3(xs)
                ys[K * (B + b) + k] = S
                for m, v in zip(rows, xs):
                    code = e4m3_encode_saturating(abs(v) / Fraction(2) ** (S - 127))
                    yT[K * r0 + k * Mg + (m - r0)] = code | (0x80 if int(x_bits[m, k]) & 0x8000 else 0)
        B += nb[g]
    return yT, ys


def nvfp4_rows(x_bits: np.ndarray):
    """NVFP4 by the FP32 steps of the recipe (numpy float32 arithmetic) with the
    nearest-value encoders above: (codes [M, K/2], E4M3 scales [M, K/16], t)."""
    M, K = x_bits.shape
    xf = (np.asarray(x_bits, np.uint32) << 16).view(np.float32)
    big = np.float32(np.finfo(np.float32).max)
    amax = np.float32(np.max(np.abs(xf))) if xf.size else np.float32(0)
    with np.errstate(over="ignore", divide="ignore"):
        t = np.float32(1) if amax == 0 else np.float32(np.float32(2688) / amax)
    if not np.isfinite(t):
        t = big
    e4 = _e4m3()
    codes = np.zeros((M, K // 2), np.uint8)
    scales = np.zeros((M, K // 16), np.uint8)
    for m in range(M):
        for j in range(K // 16):
            blk = xf[m, 16 * j:16 * j + 16]
            ab = np.float32(np.max(np.abs(blk)))
            sb = np.float32(np.float32(ab / np.float32(6)) * t)
            S = e4m3_encode_saturating(Fraction(float(sb)))
            scales[m, j] = S
            if S == 0:
                e = np.float32(0)
            else:
                with np.errstate(over="ignore"):
                    e = np.float32(t / np.float32(float(e4[S])))
                if not np.isfinite(e):
                    e = big
            for i in range(16):
                with np.errstate(over="ignore"):
                    y = np.float32(blk[i] * e)
                c = e2m1_encode(Fraction(abs(float(y)))) if np.isfinite(y) else 7
                if np.signbit(y):
                    c |= 8
                k = 16 * j + i
                codes[m, k // 2] |= c << (4 * (k & 1))
    return codes, scales, t
