"""GPU parity of the expert-grouped FP8 GEMM (forward, row layout) against the oracle.

The operands are what the path feeds the GEMM, computed by the oracle: activations are
a workload's BF16 rows through the oracle's quantize and FP8 row conversion; weights
are synthetic BF16 matrices through the oracle's FP8 row quantizer.  Floating-point
outputs are compared within a bound derived from the arithmetic:
    |y - exact| <= 2^-8 |exact| + (1 + 2^-8) (eps_dot + (K / 64) 2^-24) sum|terms| + 2^-133
where 2^-8 |exact| is half a BF16 step, (K / 64) 2^-24 the fp32 accumulation over the
64-term chunks, and eps_dot = 2^-10 the precision of one 64-term dot product inside the
matrix core (implementation-defined in the OCP MX spec; 2^-12.3 was the worst measured
on MI355X for terms spread over 27 binades).  Rows past offs[G] must stay untouched.
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
    got = bf16_to_float(y_gpu_bits)
    bound = 2.0 ** -8 * np.abs(exact) + (1 + 2.0 ** -8) * (EPS_DOT + (K / 64) * 2.0 ** -24) * absum + 2.0 ** -133
    err = np.abs(got - exact)
    ratio = err / bound
    worst = int(np.argmax(ratio))
    steps = np.abs(y_gpu_bits.astype(np.int64) - ybf.astype(np.int64))
    steps = np.where((y_gpu_bits ^ ybf) & 0x8000, 2 ** 16, steps)      # sign differs
    say(f"{what}: {err.size} outputs, worst err/bound {ratio[worst]:.3g}, "
        f"equal to the oracle's BF16 {np.mean(steps == 0):.4f}, within one step {np.mean(steps <= 1):.4f}, "
        f"max err/sum|terms| {np.max(err / np.maximum(absum, 1e-300)):.3g}")
    assert ratio[worst] <= 1.0, (what, worst, got[worst], exact[worst], absum[worst])
    assert np.mean(steps <= 1) >= 0.99, what


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
