"""GPU parity of the weight-gradient FP8 GEMM over the column layouts against the oracle.

The operands are what the path feeds this GEMM, computed by the oracle: X^T is a
workload's BF16 activations through the oracle's quantize and FP4 -> FP8 column
conversion (width K); dY^T is a BF16 gradient of width N through the oracle's backward
column quantizer.  Outputs are compared within the bound of the forward GEMM's test,
with the contraction running over an expert's tokens:
    |y - exact| <= 2^-8 |exact| + (1 + 2^-8) (eps_dot + (M_g / 64) 2^-24) sum|terms| + 2^-133
(half a BF16 step; fp32 accumulation over 64-token chunks; eps_dot = 2^-11 for the
matrix core's own rounding, measured by the zero-sum probes), and the same one-step
checks as the forward GEMM's.
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

# Allowance for the matrix core's own rounding of one dot product, relative to its
# sum|terms|: the zero-sum probes below (test_gpu_gemm.py, test_gpu_wgrad.py) measured
# at most 2^-12.48 on MI355X (two 64-term chunks, terms over 36 binades); 2^-11 leaves a
# margin of 2^1.48 (about 2.8x) over that.
EPS_DOT = 2.0 ** -11
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
    """As the forward GEMM's check: every output within the bound, and within one BF16
    step of the oracle's rounding wherever the dot-product allowance is below one step
    of |exact|."""
    got = bf16_to_float(y_bits)
    allow = (1 + 2.0 ** -8) * (EPS_DOT + (mg / 64) * 2.0 ** -24) * absum
    bound = 2.0 ** -8 * np.abs(exact) + allow + 2.0 ** -133
    err = np.abs(got - exact)
    ratio = err / bound
    worst = int(np.argmax(ratio))
    steps = np.abs(y_bits.astype(np.int64) - ybf.astype(np.int64))
    steps = np.where((y_bits ^ ybf) & 0x8000, 2 ** 16, steps)
    plain = allow < 2.0 ** -8 * np.abs(exact)
    say(f"{what}: {err.size} outputs, worst err/bound {ratio[worst]:.3g}, "
        f"equal to the oracle's BF16 {np.mean(steps == 0):.4f}, within one step {np.mean(steps <= 1):.4f}, "
        f"{np.mean(plain):.4f} without cancellation, max steps there {int(steps[plain].max(initial=0))}, "
        f"max steps at |exact| >= 2^-6 sum|terms| {int(steps[np.abs(exact) >= 2.0 ** -6 * absum].max(initial=0))}")
    assert ratio[worst] <= 1.0, (what, worst, got[worst], exact[worst], absum[worst])
    far = np.nonzero(plain & (steps > 1))[0]
    assert far.size == 0, (what, far[:5], got[far[:5]], exact[far[:5]], absum[far[:5]])
    # On these inputs the matrix core's rounding stays far below EPS_DOT: every output
    # whose sum does not cancel to below 2^-6 sum|terms| is within one BF16 step.
    far = np.nonzero((np.abs(exact) >= 2.0 ** -6 * absum) & (steps > 1))[0]
    assert far.size == 0, (what, far[:5], got[far[:5]], exact[far[:5]], absum[far[:5]])


CASES = [
    # counts, N, K, capacity slack beyond offs[G]
    ([0, 37, 300, 5, 129, 1], 256, 512, 0),     # odd rows (every byte alignment), tails, no slack
    ([128, 256], 512, 256, 3),                  # whole blocks
    ([1000], 256, 256, 0),
    ([7, 0, 290, 64, 2], 256, 256, 130),
    # a multi-step expert ending at the capacity: slices of its last step reach past the
    # end of the operand buffers, whose bytes inside them must still count
    ([200, 333], 512, 256, 0),
    ([13, 0, 1021], 256, 512, 0),
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


def test_wgrad_dot_error_probe():
    """The matrix core's own rounding over the token contraction, measured as in the
    forward GEMM's probe: one expert of 1024 tokens, token j = half + perm(i) carrying
    x_j = x_i and dy_j = -dy_i, one scale per column, so every exact dW is 0 and the GPU
    output is the rounding error alone."""
    rng = np.random.default_rng(91)
    M, N, K = 1024, 256, 256
    half = M // 2
    perm = rng.permutation(half)

    def codes(shape):
        b = rng.integers(0, 256, shape)
        return np.where((b & 0x7F) == 0x7F, b - 1, b).astype(np.uint8)

    dyT = np.zeros((N, M), np.uint8)
    xT = np.zeros((K, M), np.uint8)
    dyT[:, :half] = codes((N, half))
    xT[:, :half] = codes((K, half))
    dyT[:, half + perm] = dyT[:, :half] ^ 0x80
    xT[:, half + perm] = xT[:, :half]
    nb = M // 128
    sdyT = np.repeat(rng.integers(117, 138, (1, N)), nb, axis=0).astype(np.uint8)
    sxT = np.repeat(rng.integers(117, 138, (1, K)), nb, axis=0).astype(np.uint8)
    offs = np.array([0, M], np.int32)
    y = run_wgrad(dyT.reshape(-1), sdyT.reshape(-1), xT.reshape(-1), sxT.reshape(-1), offs, M, N, K)
    exact, ybf, absum = oracle.fp8_wgrad(dyT.reshape(-1), sdyT.reshape(-1), xT.reshape(-1), sxT.reshape(-1),
                                         offs, N, K, threads=oracle.default_threads())
    assert np.all(exact == 0)
    got = np.abs(bf16_to_float(y.reshape(-1)))
    rel = got / np.maximum(absum.reshape(-1), 1e-300)
    acc = (M / 64) * 2.0 ** -24
    say(f"wgrad dot error probe: max |dW| / sum|terms| = 2^{np.log2(max(rel.max(), 2.0 ** -200)):.2f} "
        f"(fp32 accumulation allowance 2^{np.log2(acc):.2f}, EPS_DOT 2^{np.log2(EPS_DOT):.2f}), "
        f"nonzero outputs {np.mean(got > 0):.4f}")
    assert rel.max() <= (1 + 2.0 ** -8) * (EPS_DOT + acc)
