"""GPU parity of the NVFP4 variant quantizer against the oracle: codes, E4M3 block scales
and the tensor amax byte for byte, rows past offs[G] untouched."""
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
from gpu_path import CANARY, assert_bytes_equal, assert_untouched, dev, host  # noqa: E402


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _lib():
    mx.load_library()
    oracle._load()


def gpu_nvfp4(x_bits: np.ndarray, offs: np.ndarray, amax_d=None):
    M_cap, K = x_bits.shape
    codes = torch.full((max(1, M_cap), K // 2), CANARY, dtype=torch.uint8, device="cuda")
    scales = torch.full((max(1, M_cap), K // 16), CANARY, dtype=torch.uint8, device="cuda")
    amax = amax_d if amax_d is not None else torch.full((1,), -1.0, dtype=torch.float32, device="cuda")
    x_d = dev(x_bits.view(np.int16)) if M_cap else torch.zeros((1, K), dtype=torch.int16, device="cuda")
    mx.mxfp4_nvfp4_quantize_rows(x_d, codes, scales, amax, dev(offs), M_cap=M_cap, K=K)
    torch.cuda.synchronize()
    return host(codes), host(scales), float(host(amax)[0])


def check_nvfp4(x_bits: np.ndarray, offs: np.ndarray, what: str, threads=None):
    threads = threads or oracle.default_threads()
    M_tot = int(offs[-1])
    codes, scales, amax = gpu_nvfp4(x_bits, offs)
    c_o, s_o, a_o, t_o = oracle.nvfp4_quantize_rows(x_bits, rows=M_tot, threads=threads)
    assert amax == a_o, (what, amax, a_o)
    K = x_bits.shape[1]
    assert_bytes_equal(scales[:M_tot], s_o[:M_tot], f"{what}: scales", row_len=K // 16)
    assert_bytes_equal(codes[:M_tot], c_o[:M_tot], f"{what}: codes", row_len=K // 2)
    assert_untouched(codes[M_tot:], f"{what}: codes past offs[G]")
    assert_untouched(scales[M_tot:], f"{what}: scales past offs[G]")
    return amax, t_o


SMALL = [
    ([0, 37, 300, 5], 48, "normal", 11),        # 16-blocks across MX block boundaries
    ([128, 1, 0, 255], 512, "t3", 0),
    ([3], 7168, "swiglu", 2),
    ([64, 64], 16, "normal", 0),                # one block per row
]


@pytest.mark.parametrize("counts,K,values,slack", SMALL)
def test_nvfp4_ragged(counts, K, values, slack):
    say(f"nvfp4 counts={counts} K={K} values={values}")
    seg = workloads.ragged_case(counts, K, seed=K + len(counts), values=values, M_cap=sum(counts) + slack)
    check_nvfp4(seg.x_bits, seg.offs, "ragged")


def _scaled_grid(rng, M, K):
    grid = np.array([0, 0.25, 0.5, 0.75, 1, 1.25, 1.5, 1.75, 2, 2.5, 3, 3.5, 4, 5, 6], np.float32)
    v = rng.choice(grid, (M, K)) * rng.choice([-1, 1], (M, K)).astype(np.float32)
    return v * (2.0 ** rng.integers(-3, 4, (M, K // 16))).repeat(16, axis=1).astype(np.float32)


@pytest.mark.parametrize("kind", ["grid", "wide", "tiny_tensor", "subnormal_rows", "zero"])
def test_nvfp4_value_kinds(kind):
    """Rounding ties on scaled E2M1 grids, blocks spread over 60 binades, a tensor whose
    scale quotient overflows FP32 (t = FLT_MAX), BF16 subnormal rows, an all-zero tensor."""
    rng = np.random.default_rng({"grid": 81, "wide": 82, "tiny_tensor": 83, "subnormal_rows": 84, "zero": 85}[kind])
    M, K = 96, 256
    if kind == "grid":
        v = _scaled_grid(rng, M, K)
    elif kind == "wide":
        v = rng.standard_normal((M, K)) * 2.0 ** rng.integers(-30, 30, (M, K // 16)).repeat(16, axis=1)
    elif kind == "tiny_tensor":
        v = rng.standard_normal((M, K)) * 2.0 ** -120
    elif kind == "subnormal_rows":
        v = rng.standard_normal((M, K))
        v[::7] *= 2.0 ** -130
    else:
        v = np.zeros((M, K))
    x = workloads.to_bf16_bits(np.asarray(v, np.float32))
    x[1, :16] = 0x8000                                         # a block of -0
    x[2, 16:32] |= 0x8000                                      # a negative block
    offs = np.array([0, 40, 40, M], np.int32)
    amax, t = check_nvfp4(x, offs, kind)
    if kind == "tiny_tensor":
        assert t == float(np.finfo(np.float32).max)
    if kind == "zero":
        assert amax == 0 and t == 1.0


def test_nvfp4_no_rows_resets_amax():
    x = np.zeros((0, 64), np.uint16)
    codes, scales, amax = gpu_nvfp4(x, np.zeros(3, np.int32))
    assert amax == 0.0
    x = workloads.ragged_case([5], 64, seed=3, M_cap=9).x_bits
    codes, scales, amax = gpu_nvfp4(x, np.array([0, 0], np.int32))
    assert amax == 0.0 and np.all(codes == CANARY) and np.all(scales == CANARY)


def test_nvfp4_reused_amax_buffer():
    """A second call on the same amax buffer with a smaller tensor starts from zero."""
    amax_d = torch.zeros(1, dtype=torch.float32, device="cuda")
    big = workloads.ragged_case([100], 64, seed=4).x_bits
    small = (big.astype(np.uint32) & 0x807F) | (100 << 7)        # every magnitude in [2^-27, 2^-26)
    small = small.astype(np.uint16)
    offs = np.array([0, 100], np.int32)
    _, _, a1 = gpu_nvfp4(big, offs, amax_d)
    c2, s2, a2 = gpu_nvfp4(small, offs, amax_d)
    c_o, s_o, a_o, _ = oracle.nvfp4_quantize_rows(small)
    assert a1 > a2 == a_o
    assert np.array_equal(c2, c_o) and np.array_equal(s2, s_o)


@pytest.mark.parametrize("cfg", [2, 4, 5])
def test_nvfp4_full_configs(cfg):
    threads = oracle.default_threads()
    w = workloads.make_config(cfg, 0)
    for seg in w.segments:
        say(f"nvfp4 config {cfg} {seg.name}: M_cap={seg.M_cap} K={seg.K} G={seg.G}")
        check_nvfp4(seg.x_bits, seg.offs, f"config {cfg} {seg.name}", threads=threads)


# ---- stochastic rounding of the element codes ----------------------------------------

def gpu_nvfp4_sr(x_bits: np.ndarray, offs: np.ndarray, seed: int):
    M_cap, K = x_bits.shape
    codes = torch.full((max(1, M_cap), K // 2), CANARY, dtype=torch.uint8, device="cuda")
    scales = torch.full((max(1, M_cap), K // 16), CANARY, dtype=torch.uint8, device="cuda")
    amax = torch.full((1,), -1.0, dtype=torch.float32, device="cuda")
    mx.mxfp4_nvfp4_quantize_rows_sr(dev(x_bits.view(np.int16)), codes, scales, amax, dev(offs), seed,
                                    M_cap=M_cap, K=K)
    torch.cuda.synchronize()
    return host(codes), host(scales), float(host(amax)[0])


def check_nvfp4_sr(x_bits: np.ndarray, offs: np.ndarray, seed: int, what: str, threads=None):
    threads = threads or oracle.default_threads()
    M_tot, K = int(offs[-1]), x_bits.shape[1]
    codes, scales, amax = gpu_nvfp4_sr(x_bits, offs, seed)
    c_o, s_o, a_o, _ = oracle.nvfp4_quantize_rows_sr(x_bits, seed, rows=M_tot, threads=threads)
    assert amax == a_o, (what, amax, a_o)
    assert_bytes_equal(scales[:M_tot], s_o[:M_tot], f"{what}: scales", row_len=K // 16)
    assert_bytes_equal(codes[:M_tot], c_o[:M_tot], f"{what}: codes", row_len=K // 2)
    assert_untouched(codes[M_tot:], f"{what}: codes past offs[G]")
    assert_untouched(scales[M_tot:], f"{what}: scales past offs[G]")
    return codes[:M_tot]


SEEDS = [0, 1, 0xFFFFFFFF, 0x1_0000_0000, 0xDEADBEEF_01234567, 2 ** 64 - 1]


@pytest.mark.parametrize("seed", SEEDS)
def test_nvfp4_sr_ragged_seeds(seed):
    """Both key words of the seed, odd row counts, 16-blocks across MX block boundaries."""
    say(f"nvfp4 sr seed={seed:#x}")
    seg = workloads.ragged_case([0, 37, 300, 5], 48, seed=21, M_cap=350)
    check_nvfp4_sr(seg.x_bits, seg.offs, seed, "sr ragged")


@pytest.mark.parametrize("kind", ["grid", "wide", "tiny_tensor", "subnormal_rows", "zero"])
def test_nvfp4_sr_value_kinds(kind):
    """Scaled E2M1 grids (values that must not move), 60 binades, an overflowing encode
    scale, BF16 subnormal rows, an all-zero tensor."""
    rng = np.random.default_rng({"grid": 91, "wide": 92, "tiny_tensor": 93, "subnormal_rows": 94, "zero": 95}[kind])
    M, K = 96, 256
    if kind == "grid":
        v = _scaled_grid(rng, M, K)
    elif kind == "wide":
        v = rng.standard_normal((M, K)) * 2.0 ** rng.integers(-30, 30, (M, K // 16)).repeat(16, axis=1)
    elif kind == "tiny_tensor":
        v = rng.standard_normal((M, K)) * 2.0 ** -120
    elif kind == "subnormal_rows":
        v = rng.standard_normal((M, K))
        v[::7] *= 2.0 ** -130
    else:
        v = np.zeros((M, K))
    x = workloads.to_bf16_bits(np.asarray(v, np.float32))
    x[1, :16] = 0x8000
    x[2, 16:32] |= 0x8000
    check_nvfp4_sr(x, np.array([0, 40, 40, M], np.int32), 77, f"sr {kind}")


def test_nvfp4_sr_seed_changes_codes_not_scales():
    seg = workloads.ragged_case([200], 512, seed=5)
    c1, s1, _ = gpu_nvfp4_sr(seg.x_bits, seg.offs, 1)
    c2, s2, _ = gpu_nvfp4_sr(seg.x_bits, seg.offs, 2)
    c3, _, _ = gpu_nvfp4_sr(seg.x_bits, seg.offs, 1)
    assert np.array_equal(s1, s2) and np.array_equal(c1, c3) and not np.array_equal(c1, c2)


@pytest.mark.parametrize("cfg", [2, 4, 5])
def test_nvfp4_sr_full_configs(cfg):
    threads = oracle.default_threads()
    w = workloads.make_config(cfg, 0)
    for seg in w.segments:
        say(f"nvfp4 sr config {cfg} {seg.name}: M_cap={seg.M_cap} K={seg.K} G={seg.G}")
        check_nvfp4_sr(seg.x_bits, seg.offs, 0x5EED0000 + cfg, f"sr config {cfg} {seg.name}", threads=threads)
