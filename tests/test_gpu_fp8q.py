"""GPU parity of the backward FP8 quantizer (BF16 -> E4M3FN, 1x128 blocks, UE8M0
scales), row layout and transposed column layout, against the oracle, byte for byte,
through the C ABI."""
from __future__ import annotations

import os
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

import torch  # noqa: E402

import block_scaled_precision_bf16tofp4row_amd as mx  # noqa: E402
import oracle  # noqa: E402
import workloads  # noqa: E402
from gpu_path import (assert_bytes_equal, assert_untouched, check_fp8q_cols, check_fp8q_rows,  # noqa: E402
                      dev, gpu_fp8q_cols, gpu_fp8q_rows, host)


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _lib():
    mx.load_library()          # fails loudly when the HIP library is missing
    oracle._load()


RAGGED = [
    ([0, 1, 127, 128, 129, 0, 300, 5], 512, "normal", 37),
    ([260], 128, "t3", 0),
    ([3, 0, 0, 250, 129], 2048, "swiglu", 128),
    ([1], 128, "normal", 0),
    ([0, 0, 0], 256, "normal", 64),
    ([200, 77, 513], 7168, "t3", 5),
    ([1, 383, 128], 384, "t3", 0),
    ([129, 0, 300, 256], 640, "normal", 3),        # last 256-column tile is 128 wide
]


@pytest.mark.parametrize("counts,K,values,slack", RAGGED)
def test_fp8q_rows_small_ragged(counts, K, values, slack):
    say(f"fp8q rows counts={counts} K={K} values={values} slack={slack}")
    seg = workloads.ragged_case(counts, K, seed=len(counts) + K + 1, values=values,
                                M_cap=sum(counts) + slack)
    check_fp8q_rows(seg.x_bits, seg.offs)


def _every_magnitude_blocks():
    """128-element blocks whose first element fixes the amax (every exponent field
    0..254, mantissa 0x7F or a saturation-band mantissa) and whose other 127 elements
    walk the BF16 magnitudes at or below it, alternating signs."""
    blocks = []
    for e_amax in range(0, 255):
        for top in ((0x7F, 0x68, 0x61) if e_amax >= 8 else (0x7F,)):
            amax_bits = (e_amax << 7) | top
            if e_amax in (0, 1, 8, 9, 127, 200, 254) and top == 0x7F:
                cands = np.arange(0, amax_bits + 1, dtype=np.uint32)       # the whole range
            else:
                cands = np.arange(max(0, amax_bits - 127 * 6), amax_bits + 1, dtype=np.uint32)
            n = (cands.size + 126) // 127
            body = np.zeros(n * 127, np.uint32)
            body[:cands.size] = cands
            body = body.reshape(n, 127).astype(np.uint16)
            body[:, 1::2] |= 0x8000
            blk = np.zeros((n, 128), np.uint16)
            blk[:, 0] = amax_bits | (0x8000 if e_amax % 2 else 0)
            blk[:, 1:] = body
            blocks.append(blk)
    return np.concatenate(blocks)


def test_fp8q_rows_every_bf16_magnitude():
    x = _every_magnitude_blocks()
    pad = (-x.shape[0]) % 4
    x = np.concatenate([x, np.zeros((pad, 128), np.uint16)]).reshape(-1, 512)
    say(f"exhaustive fp8q: {x.shape[0]} rows x 512")
    offs = np.array([0, x.shape[0]], np.int32)
    check_fp8q_rows(x, offs)


def test_fp8q_rows_saturation_band_every_scale():
    """Every block maximum in [448, 512) * 2^(S-127) for S = 0..246 (BF16's range):
    the saturating case the hardware convert does not handle by itself."""
    rows = []
    for e in range(8, 255):
        for mant in range(0x60, 0x80):
            blk = np.zeros(128, np.uint16)
            blk[0] = (e << 7) | mant
            blk[1] = 0x8000 | (e << 7) | mant
            blk[2] = (e << 7) | 0x5F                        # just below 448: not clamped
            blk[3:] = np.arange(3, 128, dtype=np.uint16) * 0x101 & 0x7FFF
            blk[3:] = np.minimum(blk[3:], (e << 7) | mant)
            rows.append(blk)
    x = np.stack(rows)
    pad = (-x.shape[0]) % 2
    x = np.concatenate([x, np.zeros((pad, 128), np.uint16)]).reshape(-1, 256)
    offs = np.array([0, x.shape[0]], np.int32)
    say(f"saturation band: {x.shape[0]} rows x 256")
    check_fp8q_rows(x, offs)
    y, _ = gpu_fp8q_rows(dev(x), dev(offs), x.shape[0], 256)
    y = host(y).reshape(-1, 128)
    assert np.all((y[:, 0] & 0x7F) <= 0x7E) and np.all(y[:, 1] & 0x80)


def test_fp8q_rows_no_rows_writes_nothing():
    K, M_cap = 256, 300
    x = workloads.ragged_case([0, 0], K, M_cap=M_cap).x_bits
    offs = np.zeros(3, np.int32)
    y, ys = gpu_fp8q_rows(dev(x), dev(offs), M_cap, K)
    torch.cuda.synchronize()
    assert_untouched(host(y), "y")
    assert_untouched(host(ys), "ys")


def test_fp8q_rows_side_stream_and_determinism():
    seg = workloads.ragged_case([500, 3, 700], 1024, seed=4, values="t3")
    s = torch.cuda.Stream()
    x_d, offs_d = dev(seg.x_bits), dev(seg.offs)
    s.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(2):
        with torch.cuda.stream(s):
            y, ys = gpu_fp8q_rows(x_d, offs_d, seg.M_cap, seg.K)
        s.synchronize()
        outs.append((host(y), host(ys)))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
    y_o, ys_o = oracle.fp8q_rows(seg.x_bits)
    assert_bytes_equal(outs[0][0], y_o, "fp8q rows on a side stream", row_len=seg.K)


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_fp8q_rows_full_config(cfg):
    """The row quantizer at each workload's full size (the BF16 tensor of the
    workload stands in for the gradient of the same shape), every byte compared."""
    say(f"fp8q config {cfg}: generating")
    w = workloads.make_config(cfg, 0)
    for seg in w.segments:
        say(f"fp8q config {cfg} {seg.name}: M_cap={seg.M_cap} K={seg.K} G={seg.G}")
        check_fp8q_rows(seg.x_bits, seg.offs)
        torch.cuda.empty_cache()


# ---- transposed column layout ----------------------------------------------------------

@pytest.mark.parametrize("counts,K,values,slack", RAGGED)
def test_fp8q_cols_small_ragged(counts, K, values, slack):
    say(f"fp8q cols counts={counts} K={K} values={values} slack={slack}")
    seg = workloads.ragged_case(counts, K, seed=len(counts) + K + 2, values=values,
                                M_cap=sum(counts) + slack)
    check_fp8q_cols(seg.x_bits, seg.offs)


def test_fp8q_cols_many_experts():
    """G = 300 (the strip search scans experts 64 at a time), mostly empty."""
    rng = np.random.default_rng(11)
    counts = np.zeros(300, np.int64)
    nz = rng.choice(300, 12, replace=False)
    counts[nz] = rng.integers(1, 300, size=12)
    say(f"fp8q cols G=300 nonzero={sorted(nz.tolist())}")
    seg = workloads.ragged_case(counts, 256, seed=13, values="normal", M_cap=int(counts.sum()) + 3)
    check_fp8q_cols(seg.x_bits, seg.offs)


def test_fp8q_cols_carry_across_strips():
    """Each workgroup quantizes several consecutive strips of one expert (wide K, many
    rows), so the line straddling two strips is carried; sizes 256n + r put short last
    strips behind a carried line."""
    counts = [257, 771, 514, 1025, 263, 2051, 258, 1031, 5, 270, 2307, 769, 1283, 259, 517,
              1797, 3, 261, 1539, 130]
    say(f"fp8q cols carry counts={counts} K=7168")
    seg = workloads.ragged_case(counts, 7168, seed=22, values="t3", M_cap=sum(counts) + 11)
    check_fp8q_cols(seg.x_bits, seg.offs)


def _as_column_blocks(blocks: np.ndarray, K: int) -> np.ndarray:
    """[n, 128] blocks -> an [128 m, K] matrix whose column k, rows 128b .. 128b + 127, is
    block b K + k (zero blocks pad n to a multiple of K)."""
    n = blocks.shape[0]
    m = (n + K - 1) // K
    pad = np.zeros((m * K - n, 128), np.uint16)
    b = np.concatenate([blocks, pad]).reshape(m, K, 128)
    return np.ascontiguousarray(b.transpose(0, 2, 1).reshape(128 * m, K))


def test_fp8q_cols_every_bf16_magnitude():
    x = _as_column_blocks(_every_magnitude_blocks(), 512)
    say(f"exhaustive fp8q cols: {x.shape[0]} rows x 512")
    check_fp8q_cols(x, np.array([0, x.shape[0]], np.int32))


def test_fp8q_cols_saturation_band_every_scale():
    rows = []
    for e in range(8, 255):
        for mant in range(0x60, 0x80):
            blk = np.zeros(128, np.uint16)
            blk[0] = (e << 7) | mant
            blk[1] = 0x8000 | (e << 7) | mant
            blk[2] = (e << 7) | 0x5F
            blk[3:] = np.minimum(np.arange(3, 128, dtype=np.uint16) * 0x101 & 0x7FFF, (e << 7) | mant)
            rows.append(blk)
    x = _as_column_blocks(np.stack(rows), 256)
    say(f"saturation band, columns: {x.shape[0]} rows x 256")
    check_fp8q_cols(x, np.array([0, x.shape[0]], np.int32))


def test_fp8q_cols_no_rows_writes_nothing():
    K, M_cap = 256, 300
    x = workloads.ragged_case([0, 0], K, M_cap=M_cap).x_bits
    offs = np.zeros(3, np.int32)
    yT, ys = gpu_fp8q_cols(dev(x), dev(offs), M_cap, K, 2)
    torch.cuda.synchronize()
    assert_untouched(host(yT), "yT")
    assert_untouched(host(ys), "ysT")


def test_fp8q_cols_side_stream_and_determinism():
    seg = workloads.ragged_case([500, 3, 700], 1024, seed=5, values="t3")
    s = torch.cuda.Stream()
    x_d, offs_d = dev(seg.x_bits), dev(seg.offs)
    s.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(2):
        with torch.cuda.stream(s):
            yT, ys = gpu_fp8q_cols(x_d, offs_d, seg.M_cap, seg.K, seg.G)
        s.synchronize()
        outs.append((host(yT), host(ys)))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
    yT_o, ys_o = oracle.fp8q_cols(seg.x_bits, seg.offs)
    n = seg.M_tot * seg.K
    assert_bytes_equal(outs[0][0][:n], yT_o[:n], "fp8q cols on a side stream")


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_fp8q_cols_full_config(cfg):
    """The column quantizer at each workload's full size, every byte compared."""
    say(f"fp8q cols config {cfg}: generating")
    w = workloads.make_config(cfg, 0)
    for seg in w.segments:
        say(f"fp8q cols config {cfg} {seg.name}: M_cap={seg.M_cap} K={seg.K} G={seg.G}")
        check_fp8q_cols(seg.x_bits, seg.offs)
        torch.cuda.empty_cache()
