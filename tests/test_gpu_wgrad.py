"""GPU parity of the weight-gradient FP8 GEMM over the column layouts against the oracle.

The operands are what the path feeds this GEMM, computed by the oracle: X^T is a
workload's BF16 activations through the oracle's quantize and FP4 -> FP8 column
conversion (width K); dY^T is a BF16 gradient of width N through the oracle's backward
column quantizer.  Outputs are compared within the bound of the forward GEMM's test,
with the contraction running over an expert's tokens:
    |y - exact| <= 2^-8 |exact| + (1 + 2^-8) (eps_dot + (M_g / 64) 2^-24) sum|terms| + 2^-133
(half a BF16 step; fp32 accumulation over 64-token chunks; eps_dot = 2^-10 for one
64-term dot product inside the matrix core, implementation-defined in the OCP MX spec).
Every element of dW is written, zeros for experts with no tokens.
"""
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
from gpu_path import dev, host  # noqa: E402

EPS_DOT = 2.0 ** -10
CANARY16 = 0xA5A5
CANARY8 = 0x5A


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _lib():
    mx.load_library()
    oracle._load()


def bf16_to_float(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


def in_capacity(data: np.ndarray, cap: int, fill: int = CANARY8) -> np.ndarray:
    """The oracle's layout bytes at the start of a buffer of the ABI's capacity."""
    out = np.full(max(1, cap), fill, np.uint8)
    out[: data.size] = data
    return out


def column_operands(counts, N, K, M_cap, seed, threads):
    """X^T (width K) from activations through quantize + column conversion, and dY^T
    (width N) from a gradient through the backward column quantizer, all by the oracle."""
    x = workloads.ragged_case(counts, K, seed=seed, M_cap=M_cap)
    dy = workloads.ragged_case(counts, N, seed=seed + 1, M_cap=M_cap)
    M_tot = int(x.offs[-1])
    codes, scales = oracle.quantize_rows(x.x_bits, rows=M_tot, threads=threads)
    xT, sxT = oracle.fp8_cols(codes, scales, x.offs, threads=threads)
    dyT, sdyT = oracle.fp8q_cols(dy.x_bits, x.offs, threads=threads)
    return x.offs, dyT[: N * M_tot], sdyT, xT[: K * M_tot], sxT


def run_wgrad(dyT, sdyT, xT, sxT, offs, M_cap, N, K):
    G = offs.size - 1
    cap_n = mx.mxfp4_cols_scale_capacity(M_cap, N, G)
    cap_k = mx.mxfp4_cols_scale_capacity(M_cap, K, G)
    dw = torch.full((max(1, G * N * K),), CANARY16, dtype=torch.int32, device="cuda").to(torch.int16)
    mx.mxfp4_fp8_grouped_gemm_wgrad(dev(in_capacity(dyT, N * M_cap)), dev(in_capacity(sdyT, cap_n)),
                                    dev(in_capacity(xT, K * M_cap)), dev(in_capacity(sxT, cap_k)), dw,
                                    dev(offs), N=N, K=K, G=G, M_cap=M_cap)
    torch.cuda.synchronize()
    return host(dw).view(np.uint16)[: G * N * K].reshape(G, N, K)


def check_points(y_bits, exact, ybf, absum, mg, what):
    got = bf16_to_float(y_bits)
    bound = 2.0 ** -8 * np.abs(exact) + (1 + 2.0 ** -8) * (EPS_DOT + (mg / 64) * 2.0 ** -24) * absum + 2.0 ** -133
    err = np.abs(got - exact)
    ratio = err / bound
    worst = int(np.argmax(ratio))
    steps = np.abs(y_bits.astype(np.int64) - ybf.astype(np.int64))
    steps = np.where((y_bits ^ ybf) & 0x8000, 2 ** 16, steps)
    say(f"{what}: {err.size} outputs, worst err/bound {ratio[worst]:.3g}, "
        f"equal to the oracle's BF16 {np.mean(steps == 0):.4f}, within one step {np.mean(steps <= 1):.4f}")
    assert ratio[worst] <= 1.0, (what, worst, got[worst], exact[worst], absum[worst])
    assert np.mean(steps <= 1) >= 0.99, what


CASES = [
    # counts, N, K, capacity slack beyond offs[G]
    ([0, 37, 300, 5, 129, 1], 256, 512, 0),     # odd rows (every byte alignment), tails, no slack
    ([128, 256], 512, 256, 3),                  # whole blocks
    ([1000], 256, 256, 0),
    ([7, 0, 290, 64, 2], 256, 256, 130),
]


@pytest.mark.parametrize("counts,N,K,slack", CASES)
def test_wgrad_small_every_output(counts, N, K, slack):
    threads = oracle.default_threads()
    M_cap = sum(counts) + slack
    say(f"wgrad small: counts={counts} N={N} K={K} M_cap={M_cap}")
    offs, dyT, sdyT, xT, sxT = column_operands(counts, N, K, M_cap, seed=sum(counts) + N, threads=threads)
    y = run_wgrad(dyT, sdyT, xT, sxT, offs, M_cap, N, K)
    exact, ybf, absum = oracle.fp8_wgrad(dyT, sdyT, xT, sxT, offs, N, K, threads=threads)
    mg = np.diff(offs.astype(np.int64))[:, None, None] * np.ones((1, N, K))
    check_points(y.reshape(-1), exact.reshape(-1), ybf.reshape(-1), absum.reshape(-1), mg.reshape(-1), "small")
    for g, c in enumerate(counts):
        if c == 0:
            assert np.all(y[g] == 0), g                 # an expert with no tokens: dW_g = 0


def test_wgrad_random_bytes_and_scales():
    """Operands that no quantizer produces: every E4M3 code (NaN excluded) and scale
    bytes over a range, in the column layout."""
    rng = np.random.default_rng(61)
    counts = [3, 130, 0, 255, 17]
    N, K = 256, 256
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    M = int(offs[-1])
    nb = int(sum((c + 127) // 128 for c in counts))

    def codes(n):
        b = rng.integers(0, 256, n)
        return np.where((b & 0x7F) == 0x7F, b - 1, b).astype(np.uint8)

    dyT, xT = codes(N * M), codes(K * M)
    sdyT = rng.integers(112, 140, nb * N).astype(np.uint8)
    sxT = rng.integers(112, 140, nb * K).astype(np.uint8)
    y = run_wgrad(dyT, sdyT, xT, sxT, offs, M, N, K)
    exact, ybf, absum = oracle.fp8_wgrad(dyT, sdyT, xT, sxT, offs, N, K, threads=oracle.default_threads())
    mg = np.diff(offs.astype(np.int64))[:, None, None] * np.ones((1, N, K))
    check_points(y.reshape(-1), exact.reshape(-1), ybf.reshape(-1), absum.reshape(-1), mg.reshape(-1), "random")


def test_wgrad_many_experts():
    """More than 64 experts (tiles in expert order instead of largest first), many empty."""
    rng = np.random.default_rng(62)
    counts = [int(c) if rng.random() < 0.6 else 0 for c in rng.integers(1, 160, 70)]
    N, K = 256, 256
    M_cap = sum(counts) + 17
    say(f"wgrad many experts: G={len(counts)} tokens={sum(counts)}")
    threads = oracle.default_threads()
    offs, dyT, sdyT, xT, sxT = column_operands(counts, N, K, M_cap, seed=62, threads=threads)
    y = run_wgrad(dyT, sdyT, xT, sxT, offs, M_cap, N, K)
    gs = np.repeat(np.arange(len(counts)), 40)
    ns = rng.integers(0, N, gs.size)
    ks = rng.integers(0, K, gs.size)
    exact, ybf, absum = oracle.fp8_wgrad_at(dyT, sdyT, xT, sxT, offs, N, K, gs, ns, ks, threads=threads)
    check_points(y[gs, ns, ks], exact, ybf, absum, np.diff(offs.astype(np.int64))[gs], "many experts")
    for g, c in enumerate(counts):
        if c == 0:
            assert np.all(y[g] == 0), g


def test_wgrad_no_tokens_writes_zeros():
    G, N, K = 3, 256, 256
    y = run_wgrad(np.zeros(0, np.uint8), np.zeros(0, np.uint8), np.zeros(0, np.uint8), np.zeros(0, np.uint8),
                  np.zeros(G + 1, np.int32), 0, N, K)
    assert np.all(y == 0)


def test_wgrad_full_size_sampled():
    """The weight gradient of the 8 local experts at full size: X^T of the 65536 routed
    rows x hidden 7168 and dY^T of a [65536, 4096] gradient (the fused gate and up
    projections); sampled outputs, every expert's corners and tile edges included."""
    threads = oracle.default_threads()
    w5 = workloads.make_config(5, 0)
    seg = w5.segments[0]
    N, K, G = 4096, seg.K, seg.G
    M_cap, M_tot = seg.M_cap, seg.M_tot
    say(f"wgrad full size: M_cap={M_cap} K={K} N={N} G={G}: preparing operands")
    codes, scales = oracle.quantize_rows(seg.x_bits, rows=M_tot, threads=threads)
    xT, sxT = oracle.fp8_cols(codes, scales, seg.offs, threads=threads)
    del codes, scales
    grad = workloads.ragged_case(np.diff(seg.offs.astype(np.int64)), N, seed=11, M_cap=M_cap)
    dyT, sdyT = oracle.fp8q_cols(grad.x_bits, seg.offs, threads=threads)
    del grad
    say("wgrad full size: running")
    y = run_wgrad(dyT[: N * M_tot], sdyT, xT[: K * M_tot], sxT, seg.offs, M_cap, N, K)
    rng = np.random.default_rng(4)
    gs = list(rng.integers(0, G, 3000))
    ns = list(rng.integers(0, N, 3000))
    ks = list(rng.integers(0, K, 3000))
    for g in range(G):
        for n in (0, 255, 256, N - 1):
            for k in (0, 255, 256, K - 1):
                gs.append(g), ns.append(n), ks.append(k)
    gs, ns, ks = (np.array(v, np.int64) for v in (gs, ns, ks))
    exact, ybf, absum = oracle.fp8_wgrad_at(dyT, sdyT, xT, sxT, seg.offs, N, K, gs, ns, ks, threads=threads)
    mg = np.diff(seg.offs.astype(np.int64))[gs]
    check_points(y[gs, ns, ks], exact, ybf, absum, mg, "full size")
    for g in range(G):
        if seg.offs[g + 1] == seg.offs[g]:
            assert np.all(y[g] == 0), g
