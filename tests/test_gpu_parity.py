"""GPU parity: the HIP path (through the C ABI) against the CPU oracle, byte for
byte (codes, UE8M0 scales, E4M3 bytes, transposed outputs), plus canary checks
that nothing outside the documented output ranges is written.

Method: "Practical FP4 Training for Large-Scale MoE Models on Hopper GPUs",
technical summary section 2, items 1-3.  Tolerance: none -- every output is an
integer code decided by exact arithmetic on both sides.
"""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import block_scaled_precision_bf16tofp4row_amd as mx  # noqa: E402
import oracle  # noqa: E402
import workloads  # noqa: E402
from gpu_path import (CANARY, assert_bytes_equal, assert_untouched, check_chain, dev,  # noqa: E402
                      gpu_cols, gpu_quantize, gpu_rows, host)


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _lib():
    mx.load_library()          # fails loudly when the HIP library is missing
    oracle._load()


# ---- small ragged cases spanning several tiles with partial tails ---------------------

RAGGED = [
    ([0, 1, 127, 128, 129, 0, 300, 5], 512, "normal", 37),
    ([260], 128, "t3", 0),
    ([3, 0, 0, 250, 129], 2048, "swiglu", 128),
    ([1], 128, "normal", 0),
    ([0, 0, 0], 256, "normal", 64),                 # no rows at all, capacity left over
    ([200, 77, 513], 7168, "t3", 5),
    ([129, 0, 300, 256], 640, "normal", 3),        # last 256-column tile is 128 wide
    ([1, 383, 128], 384, "t3", 0),
]


@pytest.mark.parametrize("counts,K,values,slack", RAGGED)
def test_small_ragged_chain(counts, K, values, slack):
    say(f"ragged counts={counts} K={K} values={values} slack={slack}")
    M_tot = sum(counts)
    seg = workloads.ragged_case(counts, K, seed=len(counts) + K, values=values, M_cap=M_tot + slack)
    check_chain(seg.x_bits, seg.offs)


@pytest.mark.parametrize("K", [32, 96, 160, 416])
def test_quantize_ragged_k_not_multiple_of_128(K):
    """The quantizer accepts any K that is a multiple of 32 (one MX block): K of one,
    three, five and thirteen blocks, ragged experts (empty ones, single rows, partial
    tails), capacity slack past offs[G] that must keep its canary."""
    counts = [0, 1, 127, 3, 300, 0, 65, 2]
    say(f"quantize counts={counts} K={K}")
    seg = workloads.ragged_case(counts, K, seed=K, values="t3", M_cap=sum(counts) + 9)
    check_chain(seg.x_bits, seg.offs, kernels=("quantize",))


def test_many_experts_scan_chunks():
    """G = 300 (the tile search scans experts 64 at a time), mostly empty."""
    rng = np.random.default_rng(1)
    counts = np.zeros(300, np.int64)
    nz = rng.choice(300, 12, replace=False)
    counts[nz] = rng.integers(1, 300, size=12)
    say(f"G=300 nonzero={sorted(nz.tolist())}")
    seg = workloads.ragged_case(counts, 256, seed=3, values="normal", M_cap=int(counts.sum()) + 3)
    check_chain(seg.x_bits, seg.offs)


def test_cols_carry_across_strips():
    """Wide K (56 column tiles) and enough rows that each workgroup of the column
    kernel converts several consecutive 256-row strips of one expert, so the chunk
    straddling two strips is carried; expert sizes 256n + r with small r put short
    last strips (r rows) behind a carried chunk."""
    counts = [257, 771, 514, 1025, 263, 2051, 258, 1031, 5, 270, 2307, 769, 1283, 259, 517,
              1797, 3, 261, 1539, 130]
    say(f"carry counts={counts} K=7168")
    seg = workloads.ragged_case(counts, 7168, seed=21, values="t3", M_cap=sum(counts) + 11)
    check_chain(seg.x_bits, seg.offs, kernels=("quantize", "cols"))


def test_cols_aligned_experts_without_lead_in():
    """Experts whose row counts are multiples of 128 carry nothing across strips, so a
    workgroup range starting inside one needs no lead-in strip: ranges start inside
    such experts (56 column tiles, a few parts each), next to ragged ones whose ranges
    still take a lead-in; the backward column quantizer and its both-layouts mode take
    the same rule."""
    from gpu_path import check_fp8q_both, check_fp8q_cols
    counts = [2048, 1280, 131, 3072, 640, 1025, 1024, 0, 384]
    say(f"aligned experts counts={counts} K=7168")
    seg = workloads.ragged_case(counts, 7168, seed=23, values="t3", M_cap=sum(counts) + 5)
    check_chain(seg.x_bits, seg.offs, kernels=("quantize", "cols"))
    check_fp8q_cols(seg.x_bits, seg.offs)
    check_fp8q_both(seg.x_bits, seg.offs)


@pytest.mark.parametrize("counts,K", [
    ([4096, 0, 8192, 4096, 0], 7168),              # 28 tiles x 9 parts: strips dealt 9 apart
    ([4096, 0, 8192, 4096, 0], 2048),
    ([0, 12288, 4096], 384),                       # last tile 128 wide; one strip per part
])
def test_cols_dealt_strips(counts, K):
    """Every expert's row count a multiple of 4096: the column kernels deal a tile's strips
    to its workgroups in turn (part, part + parts, ...) instead of contiguous ranges, each
    strip written alone (empty experts, capacity slack past offs[G], a narrow last tile);
    the backward column quantizer and its both-layouts mode take the same rule."""
    from gpu_path import check_fp8q_both, check_fp8q_cols
    say(f"dealt strips counts={counts} K={K}")
    seg = workloads.ragged_case(counts, K, seed=K + len(counts), values="t3", M_cap=sum(counts) + 7)
    check_chain(seg.x_bits, seg.offs, kernels=("quantize", "cols"))
    check_fp8q_cols(seg.x_bits, seg.offs)
    check_fp8q_both(seg.x_bits, seg.offs)


def test_cols_dealt_strips_many_experts():
    """G = 300, five experts of 4096 rows and the rest empty: dealt strips walk across
    the 64-expert chunks of the expert scan, many steps at a time, and the workgroups
    past the segment's 160 strips (256 parts of the one tile) get none."""
    from gpu_path import check_fp8q_cols
    counts = np.zeros(300, np.int64)
    counts[[3, 70, 71, 200, 299]] = 4096
    say("dealt strips G=300")
    seg = workloads.ragged_case(counts, 256, seed=5, values="normal", M_cap=int(counts.sum()))
    check_chain(seg.x_bits, seg.offs, kernels=("quantize", "cols"))
    check_fp8q_cols(seg.x_bits, seg.offs)


def test_config1_full_chain():
    w = workloads.config1(0)
    seg = w.segments[0]
    check_chain(seg.x_bits, seg.offs)


# ---- exhaustive element coverage -------------------------------------------------------

def test_quantize_every_bf16_magnitude():
    """Blocks whose first element fixes amax (exponent field 0..254) and whose other
    31 elements walk every BF16 magnitude at or below it, both signs."""
    blocks = []
    for e_amax in range(0, 255, 1):
        amax_bits = (e_amax << 7) | 0x7F
        lo = max(0, amax_bits - 31 * 40)           # dense near the top of the range
        cands = np.arange(lo, amax_bits + 1, dtype=np.uint32)
        if e_amax in (0, 1, 2, 3, 4, 127, 200, 254):
            cands = np.arange(0, amax_bits + 1, dtype=np.uint32)   # the whole range
        n = (cands.size + 30) // 31
        body = np.zeros(n * 31, np.uint32)
        body[:cands.size] = cands
        body = body.reshape(n, 31).astype(np.uint16)
        body[:, 1::2] |= 0x8000
        blk = np.zeros((n, 32), np.uint16)
        blk[:, 0] = amax_bits | (0x8000 if e_amax % 2 else 0)
        blk[:, 1:] = body
        blocks.append(blk)
    allb = np.concatenate(blocks)
    pad = (-allb.shape[0]) % 4
    allb = np.concatenate([allb, np.zeros((pad, 32), np.uint16)])
    x = allb.reshape(-1, 128)
    say(f"exhaustive quantize: {x.shape[0]} rows x 128")
    offs = np.array([0, x.shape[0]], np.int32)
    check_chain(x, offs)


def _codes_scales_all_gaps(M, K, seed):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, size=(M, K // 2), dtype=np.uint16).astype(np.uint8)
    S = rng.integers(0, 255, size=(M, K // 128))
    gaps = rng.integers(0, 255, size=(M, K // 32))
    small = rng.random((M, K // 32)) < 0.6
    gaps[small] = rng.integers(0, 16, size=int(small.sum()))
    gaps = np.minimum(gaps, np.repeat(S, 4, axis=1))
    gaps.reshape(-1, 4)[:, 0] = 0
    scales = (np.repeat(S, 4, axis=1) - gaps).astype(np.uint8)
    return codes, scales


def test_rows_every_gap():
    M, K = 1000, 1024
    codes, scales = _codes_scales_all_gaps(M, K, 7)
    offs = np.array([0, M], np.int32)
    y_d, ys_d = gpu_rows(dev(codes), dev(scales), dev(offs), M, K)
    y_o, ys_o = oracle.fp8_rows(codes, scales, threads=oracle.default_threads())
    assert_bytes_equal(host(y_d), y_o, "fp8 rows", row_len=K)
    assert_bytes_equal(host(ys_d), ys_o, "fp8 row scales", row_len=K // 128)


def test_cols_every_gap():
    """Row scales spread over the whole UE8M0 range so column blocks see every gap."""
    rng = np.random.default_rng(8)
    counts = [130, 0, 257, 1, 128]
    M, K = sum(counts), 512
    offs = workloads.offsets_from_counts(counts)
    codes = rng.integers(0, 256, size=(M, K // 2), dtype=np.uint16).astype(np.uint8)
    scales = rng.integers(0, 255, size=(M, K // 32)).astype(np.uint8)
    near = rng.random(M) < 0.5
    scales[near] = (200 - rng.integers(0, 16, size=(int(near.sum()), K // 32))).astype(np.uint8)
    G = len(counts)
    yT_d, ys_d = gpu_cols(dev(codes), dev(scales), dev(offs), M, K, G)
    used = oracle.cols_scale_size(offs, K)
    yT_o, ys_o = oracle.fp8_cols(codes, scales, offs, threads=oracle.default_threads())
    assert_bytes_equal(host(yT_d), yT_o, "fp8 cols")
    assert_bytes_equal(host(ys_d)[:used], ys_o[:used], "fp8 col scales")
    assert_untouched(host(ys_d)[used:], "col scales past the used blocks")


# ---- degenerate offsets, streams, determinism -----------------------------------------

def test_no_rows_writes_nothing():
    K, M_cap = 256, 300
    x = workloads.ragged_case([0, 0], K, M_cap=M_cap).x_bits
    offs = np.zeros(3, np.int32)
    offs_d = dev(offs)
    c, s = gpu_quantize(x, offs, offs_d=offs_d)
    y, ys = gpu_rows(c, s, offs_d, M_cap, K)
    yT, ysT = gpu_cols(c, s, offs_d, M_cap, K, 2)
    torch.cuda.synchronize()
    for name, t in (("codes", c), ("scales", s), ("y", y), ("ys", ys), ("yT", yT), ("ysT", ysT)):
        assert_untouched(host(t), name)


def test_side_stream_and_determinism():
    seg = workloads.ragged_case([500, 3, 700], 1024, seed=4, values="t3")
    s = torch.cuda.Stream()
    offs_d = dev(seg.offs)
    x_d = dev(seg.x_bits)
    outs = []
    s.wait_stream(torch.cuda.current_stream())
    for _ in range(2):
        with torch.cuda.stream(s):
            c, sc = gpu_quantize(seg.x_bits, seg.offs, x_d=x_d, offs_d=offs_d)
            y, ys = gpu_rows(c, sc, offs_d, seg.M_cap, seg.K)
            yT, ysT = gpu_cols(c, sc, offs_d, seg.M_cap, seg.K, seg.G)
        s.synchronize()
        outs.append([host(t) for t in (c, sc, y, ys, yT, ysT)])
    for a, b in zip(*outs):
        assert np.array_equal(a, b)
    c_o, s_o = oracle.quantize_rows(seg.x_bits)
    assert_bytes_equal(outs[0][0], c_o, "codes on a side stream")


def test_validate_offsets():
    good = dev(np.array([0, 3, 3, 10], np.int32))
    assert mx.mxfp4_validate_offsets(good, M_cap=10)
    assert not mx.mxfp4_validate_offsets(good, M_cap=9)
    assert not mx.mxfp4_validate_offsets(dev(np.array([0, 5, 4], np.int32)), M_cap=10)
    assert not mx.mxfp4_validate_offsets(dev(np.array([1, 5], np.int32)), M_cap=10)


# ---- the five workloads at full size, every byte compared ------------------------------

@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_full_config(cfg):
    say(f"config {cfg}: generating")
    w = workloads.make_config(cfg, 0)
    for seg in w.segments:
        say(f"config {cfg} {seg.name}: M_cap={seg.M_cap} K={seg.K} G={seg.G} kernels={w.kernels}")
        kernels = ("quantize",) + tuple(k for k in w.kernels if k != "quantize")
        check_chain(seg.x_bits, seg.offs, kernels=kernels)
        torch.cuda.empty_cache()
