"""GPU parity of the backward FP8 quantizer writing both layouts from one read
(mxfp4_bf16_to_fp8_rows_cols_ragged): every byte of both outputs against the oracle's
row and column quantizers, on the cases of the separate quantizers' tests."""
from __future__ import annotations

import os
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

import block_scaled_precision_bf16tofp4row_amd as mx  # noqa: E402
import oracle  # noqa: E402
import workloads  # noqa: E402
from gpu_path import check_fp8q_both  # noqa: E402
from test_gpu_fp8q import RAGGED, _as_column_blocks, _every_magnitude_blocks  # noqa: E402


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _lib():
    mx.load_library()
    oracle._load()


@pytest.mark.parametrize("counts,K,values,slack", RAGGED)
def test_both_small_ragged(counts, K, values, slack):
    say(f"fp8q both counts={counts} K={K} values={values}")
    seg = workloads.ragged_case(counts, K, seed=K + len(counts) + 1, values=values, M_cap=sum(counts) + slack)
    check_fp8q_both(seg.x_bits, seg.offs)


def test_both_many_experts():
    rng = np.random.default_rng(12)
    counts = np.zeros(300, np.int64)
    nz = rng.choice(300, 12, replace=False)
    counts[nz] = rng.integers(1, 300, size=12)
    seg = workloads.ragged_case(counts, 256, seed=14, values="normal", M_cap=int(counts.sum()) + 3)
    check_fp8q_both(seg.x_bits, seg.offs)


def test_both_carry_across_strips():
    counts = [257, 771, 514, 1025, 263, 2051, 258, 1031, 5, 270, 2307, 769, 1283, 259, 517,
              1797, 3, 261, 1539, 130]
    seg = workloads.ragged_case(counts, 7168, seed=23, values="t3", M_cap=sum(counts) + 11)
    check_fp8q_both(seg.x_bits, seg.offs)


def test_both_every_bf16_magnitude():
    """Every BF16 magnitude under every amax exponent, as column blocks; the row blocks
    of the same matrix mix them."""
    x = _as_column_blocks(_every_magnitude_blocks(), 512)
    check_fp8q_both(x, np.array([0, x.shape[0]], np.int32))


def test_both_no_rows_writes_nothing():
    x = workloads.ragged_case([4], 256, seed=5, M_cap=40).x_bits
    check_fp8q_both(x, np.array([0, 0, 0], np.int32))


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_both_full_config(cfg):
    threads = oracle.default_threads()
    w = workloads.make_config(cfg, 0)
    for seg in w.segments:
        say(f"fp8q both config {cfg} {seg.name}: M_cap={seg.M_cap} K={seg.K} G={seg.G}")
        check_fp8q_both(seg.x_bits, seg.offs, threads=threads)
