"""Seeded random ragged segments through the conversion path (quantize, row and column
conversion) and the backward FP8 quantizer (rows, columns, both layouts), each compared
byte for byte with the oracle, with canaries past every output range: expert counts
from skewed multinomials, sparse and equal splits, 1 to 300 experts, widths from 128
to 3072 (odd multiples of 128 give the narrow last column tile), capacity slack from
none to past a strip, and the three value distributions of the workloads; and segments
whose experts are all multiples of 4096 rows, whose strips the column kernels deal to
their workgroups in turn."""
from __future__ import annotations

import os
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import block_scaled_precision_bf16tofp4row_amd as mx  # noqa: E402
import workloads  # noqa: E402
from gpu_path import check_chain, check_fp8q_both, check_fp8q_cols, check_fp8q_rows  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _lib():
    mx.load_library()


def random_case(rng):
    G = int(rng.choice([1, 2, 3, 5, 8, 17, 33, 64, 65, 130, 300]))
    kind = int(rng.integers(0, 4))
    budget = int(rng.integers(1, 6000))
    if kind == 0:
        counts = rng.multinomial(budget, rng.dirichlet(np.full(G, 0.3)))
    elif kind == 1:
        counts = rng.integers(0, 3, G) * rng.integers(0, 300, G)
    elif kind == 2:
        counts = rng.integers(0, 200, G)
        counts[rng.random(G) < 0.4] = 0
    else:
        counts = np.full(G, budget // G)
        counts[rng.integers(0, G)] += budget % G
    counts = counts.astype(np.int64)
    while counts.sum() > 6000:
        counts //= 2
    K = 128 * int(rng.integers(1, 25))
    slack = int(rng.choice([0, 0, 1, 7, 127, 128, 300]))
    if counts.sum() + slack == 0:
        slack = 1
    values = str(rng.choice(["normal", "t3", "swiglu"]))
    return counts, K, slack, values, int(rng.integers(0, 1 << 30))


@pytest.mark.parametrize("seed", range(12))
def test_random_ragged_segments(seed):
    rng = np.random.default_rng(1000 + seed)
    for case in range(5):
        counts, K, slack, values, vseed = random_case(rng)
        print(f"seed {seed} case {case}: G={counts.size} M_tot={int(counts.sum())} K={K} slack={slack} "
              f"values={values} counts[:8]={counts[:8].tolist()}", flush=True)
        seg = workloads.ragged_case(counts.tolist(), K, seed=vseed, values=values,
                                    M_cap=int(counts.sum()) + slack)
        check_chain(seg.x_bits, seg.offs)
        check_fp8q_rows(seg.x_bits, seg.offs)
        check_fp8q_cols(seg.x_bits, seg.offs)
        check_fp8q_both(seg.x_bits, seg.offs)
        mx.mxfp4_wait_status()


def random_dealt_case(rng):
    """Every expert a multiple of 4096 rows (some empty): the column kernels' dealt strips."""
    G = int(rng.choice([1, 2, 3, 5, 9, 70]))
    counts = 4096 * rng.integers(0, 3, G)
    if counts.sum() == 0:
        counts[rng.integers(0, G)] = 4096
    while counts.sum() > 16384:
        counts[int(np.argmax(counts))] -= 4096
    K = 128 * int(rng.integers(1, 25))
    slack = int(rng.choice([0, 1, 128, 4096]))
    values = str(rng.choice(["normal", "t3", "swiglu"]))
    return counts.astype(np.int64), K, slack, values, int(rng.integers(0, 1 << 30))


@pytest.mark.parametrize("seed", range(4))
def test_random_dealt_segments(seed):
    rng = np.random.default_rng(2000 + seed)
    for case in range(3):
        counts, K, slack, values, vseed = random_dealt_case(rng)
        print(f"dealt seed {seed} case {case}: G={counts.size} M_tot={int(counts.sum())} K={K} slack={slack} "
              f"values={values} counts[:8]={counts[:8].tolist()}", flush=True)
        seg = workloads.ragged_case(counts.tolist(), K, seed=vseed, values=values,
                                    M_cap=int(counts.sum()) + slack)
        check_chain(seg.x_bits, seg.offs, kernels=("quantize", "cols"))
        check_fp8q_cols(seg.x_bits, seg.offs)
        check_fp8q_both(seg.x_bits, seg.offs)
        mx.mxfp4_wait_status()
