"""GPU parity of the expert-grouped FP8 GEMM (forward, row layout) against the oracle.

The operands are what the path feeds the GEMM, computed by the oracle: activations are
a workload's BF16 rows through the oracle's quantize and FP8 row conversion; weights
are synthetic BF16 matrices through the oracle's FP8 row quantizer.  Floating-point
outputs are compared within a bound derived from the arithmetic:
    |y - exact| <= 2^-8 |exact| + (1 + 2^-8) (eps_dot + (K / 64) 2^-24) sum|terms| + 2^-133
where 2^-8 |exact| is half a BF16 step, (K / 64) 2^-24 the fp32 accumulation over the
64-term chunks, and eps_dot = 2^-11 the allowance for the matrix core's own rounding of
a dot product (implementation-defined in the OCP MX spec): the zero-sum probe at the end
of this file measures it, 2^-12.48 at worst on MI355X, and the allowance keeps a margin
of about 2.8x over that.  Beyond the bound, every output is within one BF16 step of the
oracle's rounding where the bound's dot-product allowance is below one step of |exact|,
and (a property of these inputs, whose rounding stays far below the allowance) wherever
|exact| >= 2^-6 sum|terms|.  Rows past offs[G] must stay untouched.
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


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _lib():
    mx.load_library()
    oracle._load()


def bf16_to_float(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


def activations(x_bits, M_tot, threads):
    codes, scales = oracle.quantize_rows(x_bits, rows=M_tot, threads=threads)
    a, sa = oracle.fp8_rows(codes, scales, rows=M_tot, threads=threads)
    return a, sa


def weights(G, N, K, seed, threads):
    rng = np.random.default_rng(seed)
    wb = workloads.to_bf16_bits((rng.standard_normal((G * N, K)) * 0.05).astype(np.float32))
    w, sw = oracle.fp8q_rows(wb, threads=threads)
    return w.reshape(G, N, K), sw.reshape(G, N, K // 128)


def run_gemm(a, sa, w, sw, offs, M_cap):
    G, N, K = w.shape
    y = torch.full((M_cap, N), CANARY16, dtype=torch.int32, device="cuda").to(torch.int16)
    mx.mxfp4_fp8_grouped_gemm(dev(a), dev(sa), dev(w), dev(sw), y, dev(offs), G=G, M_cap=M_cap, N=N, K=K)
    torch.cuda.synchronize()
    return host(y).view(np.uint16)


def check_points(y_gpu_bits, exact, ybf, absum, K, what):
    """Every output within the error bound, and within one BF16 step of the oracle's
    rounding of the exact value wherever the bound's dot-product allowance is below
    one step of |exact| (a difference d < 2^-8 |exact| moves the rounding by at most
    one step); elsewhere the sum cancels and only the bound applies."""
    got = bf16_to_float(y_gpu_bits)
    allow = (1 + 2.0 ** -8) * (EPS_DOT + (K / 64) * 2.0 ** -24) * absum
    bound = 2.0 ** -8 * np.abs(exact) + allow + 2.0 ** -133
    err = np.abs(got - exact)
    ratio = err / bound
    worst = int(np.argmax(ratio))
    steps = np.abs(y_gpu_bits.astype(np.int64) - ybf.astype(np.int64))
    steps = np.where((y_gpu_bits ^ ybf) & 0x8000, 2 ** 16, steps)      # sign differs
    plain = allow < 2.0 ** -8 * np.abs(exact)
    say(f"{what}: {err.size} outputs, worst err/bound {ratio[worst]:.3g}, "
        f"equal to the oracle's BF16 {np.mean(steps == 0):.4f}, within one step {np.mean(steps <= 1):.4f}, "
        f"max err/sum|terms| {np.max(err / np.maximum(absum, 1e-300)):.3g}, "
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
    ([0, 37, 300, 5], 512, 512, 11),          # empty expert, partial tiles, a 2-tile expert
    ([256], 256, 128, 0),                     # one full tile, a single K step
    ([1, 0, 513], 768, 1024, 7),              # one-row expert, tiles 256 + 256 + 1
    ([300, 45], 256, 7296, 3),                # K past the fast path's staged scales: general kernel
    ([130], 512, 384, 0),                     # K not a multiple of 256: general kernel
]


@pytest.mark.parametrize("counts,N,K,slack", CASES)
def test_gemm_small_every_output(counts, N, K, slack):
    say(f"gemm counts={counts} N={N} K={K}")
    threads = oracle.default_threads()
    M_tot = sum(counts)
    seg = workloads.ragged_case(counts, K, seed=len(counts) + N, values="normal", M_cap=M_tot + slack)
    a, sa = activations(seg.x_bits, M_tot, threads)
    w, sw = weights(len(counts), N, K, seed=K + N, threads=threads)
    y = run_gemm(a, sa, w, sw, seg.offs, seg.M_cap)
    exact, ybf, absum = oracle.fp8_gemm(a, sa, w, sw, seg.offs, threads=threads)
    check_points(y[:M_tot].reshape(-1), exact.reshape(-1), ybf.reshape(-1), absum.reshape(-1), K, "small")
    assert np.all(y[M_tot:] == CANARY16), "rows past offs[G] were written"


def test_gemm_as_dgrad():
    """The activation gradient dX[m, k] = sum_n dY[m, n] W_g[n, k] through the same entry
    point: A = the backward row quantizer's output of an [M, N] gradient (1x128 blocks
    along N), and each expert's weight transposed to [K, N] and quantized along N."""
    threads = oracle.default_threads()
    counts, N, K = [0, 37, 300, 5], 768, 512
    M_tot = sum(counts)
    say(f"gemm as dgrad: counts={counts} N={N} K={K}")
    grad = workloads.ragged_case(counts, N, seed=21, M_cap=M_tot + 5)
    a, sa = oracle.fp8q_rows(grad.x_bits, rows=M_tot, threads=threads)
    wT, swT = weights(len(counts), K, N, seed=22, threads=threads)       # W_g^T [K, N]
    y = run_gemm(a, sa, wT, swT, grad.offs, grad.M_cap)
    exact, ybf, absum = oracle.fp8_gemm(a, sa, wT, swT, grad.offs, threads=threads)
    check_points(y[:M_tot].reshape(-1), exact.reshape(-1), ybf.reshape(-1), absum.reshape(-1), N, "dgrad")
    assert np.all(y[M_tot:] == CANARY16), "rows past offs[G] were written"


def test_gemm_many_experts():
    """300 experts, 12 of them with tokens (the tile -> expert walk over many groups)."""
    threads = oracle.default_threads()
    rng = np.random.default_rng(12)
    counts = [0] * 300
    for g in rng.choice(300, 12, replace=False):
        counts[int(g)] = int(rng.integers(1, 300))
    N, K = 256, 256
    M_tot = sum(counts)
    seg = workloads.ragged_case(counts, K, seed=13, values="normal", M_cap=M_tot + 4)
    a, sa = activations(seg.x_bits, M_tot, threads)
    w, sw = weights(300, N, K, seed=14, threads=threads)
    y = run_gemm(a, sa, w, sw, seg.offs, seg.M_cap)
    exact, ybf, absum = oracle.fp8_gemm(a, sa, w, sw, seg.offs, threads=threads)
    check_points(y[:M_tot].reshape(-1), exact.reshape(-1), ybf.reshape(-1), absum.reshape(-1), K, "300 experts")
    assert np.all(y[M_tot:] == CANARY16)


def test_gemm_no_rows_writes_nothing():
    G, N, K, M_cap = 3, 256, 256, 100
    a = np.zeros((M_cap, K), np.uint8)
    sa = np.zeros((M_cap, K // 128), np.uint8)
    w = np.zeros((G, N, K), np.uint8)
    sw = np.zeros((G, N, K // 128), np.uint8)
    y = run_gemm(a, sa, w, sw, np.zeros(G + 1, np.int32), M_cap)
    assert np.all(y == CANARY16)


def test_gemm_full_size_sampled():
    """The forward expert GEMM at full size: the 65536 routed rows x hidden 7168 of the
    8-local-expert workload against 8 experts' [4096, 7168] weights; sampled outputs
    (random points plus every expert's first and last rows and tile edges)."""
    threads = oracle.default_threads()
    w5 = workloads.make_config(5, 0)
    seg = w5.segments[0]
    N = 4096
    K = seg.K
    say(f"gemm full size: M_cap={seg.M_cap} K={K} N={N} G={seg.G}: preparing operands")
    a, sa = activations(seg.x_bits, seg.M_tot, threads)
    w, sw = weights(seg.G, N, K, seed=5, threads=threads)
    say("gemm full size: running")
    y = run_gemm(a, sa, w, sw, seg.offs, seg.M_cap)
    rng = np.random.default_rng(3)
    ms = list(rng.integers(0, seg.M_tot, 3000))
    for g in range(seg.G):
        r0, r1 = int(seg.offs[g]), int(seg.offs[g + 1])
        if r1 > r0:
            ms += [r0, r1 - 1] + [m for m in range(r0 + 255, r1, 256)][:8] + [m for m in range(r0 + 256, r1, 256)][:8]
    ms = np.array(ms, np.int64)
    ns = rng.integers(0, N, ms.size).astype(np.int64)
    ns[: seg.G * 2] = N - 1
    exact, ybf, absum = oracle.fp8_gemm_at(a, sa, w, sw, seg.offs, ms, ns, threads=threads)
    check_points(y[ms, ns], exact, ybf, absum, K, "full size")
    assert np.all(y[seg.M_tot:] == CANARY16)


def e4m3_codes(rng, shape):
    """Random E4M3FN bytes over the whole format (both signs, zeros, subnormals, up to
    448), NaN bytes excluded."""
    b = rng.integers(0, 256, shape)
    return np.where((b & 0x7F) == 0x7F, b - 1, b).astype(np.uint8)


@pytest.mark.parametrize("K", [128, 1024, 7168])
def test_gemm_dot_error_probe(K):
    """The matrix core's own rounding, measured: each product in the first half of K
    is cancelled exactly by one in the second half (a_j = a_i, w_j = -w_i under a random
    matching, so the two lie in different 64-term chunks and no chunk mirrors another;
    one scale per row, so equal bytes give equal terms).  Every exact output is then 0
    and the GPU output is the accumulated rounding error alone, which must stay within
    (EPS_DOT + (K / 64) 2^-24) sum|terms|.  E4M3 bytes over the whole format spread the
    terms of one output over up to 36 binades, the case where aligning them inside the
    matrix core loses the most."""
    rng = np.random.default_rng(K)
    M, N, half = 512, 256, K // 2
    perm = rng.permutation(half)
    a = np.zeros((M, K), np.uint8)
    w2 = np.zeros((N, K), np.uint8)
    a[:, :half] = e4m3_codes(rng, (M, half))
    w2[:, :half] = e4m3_codes(rng, (N, half))
    a[:, half + perm] = a[:, :half]
    w2[:, half + perm] = w2[:, :half] ^ 0x80
    w = w2.reshape(1, N, K)
    sa = np.repeat(rng.integers(117, 138, (M, 1)), K // 128, axis=1).astype(np.uint8)
    sw = np.repeat(rng.integers(117, 138, (1, N, 1)), K // 128, axis=2).astype(np.uint8)
    offs = np.array([0, M], np.int32)
    y = run_gemm(a, sa, w, sw, offs, M)
    exact, ybf, absum = oracle.fp8_gemm(a, sa, w, sw, offs, threads=oracle.default_threads())
    assert np.all(exact == 0)
    got = np.abs(bf16_to_float(y.reshape(-1)))
    rel = got / np.maximum(absum.reshape(-1), 1e-300)
    acc = (K / 64) * 2.0 ** -24
    say(f"dot error probe K={K}: max |y| / sum|terms| = 2^{np.log2(max(rel.max(), 2.0 ** -200)):.2f} "
        f"(fp32 accumulation allowance 2^{np.log2(acc):.2f}, EPS_DOT 2^{np.log2(EPS_DOT):.2f}), "
        f"nonzero outputs {np.mean(got > 0):.4f}")
    assert rel.max() <= (1 + 2.0 ** -8) * (EPS_DOT + acc)
