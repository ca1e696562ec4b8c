"""Seeded synthetic inputs for the BF16 -> MXFP4 -> FP8 path.

This module only draws inputs: BF16 activation matrices (as raw uint16 bits)
and int32 per-expert row offsets.  It holds none of the method's arithmetic
(no scales, no rounding to FP4/FP8), so both the oracle side and the HIP side
can take their inputs from it.

Shapes follow the DeepSeek-V3-style MoE the method is evaluated on
("Practical FP4 Training for Large-Scale MoE Models on Hopper GPUs", technical
summary section 4, Results: 671B MoE in the DeepSeek-V3 configuration): hidden
size 7168, MoE intermediate size 2048, 256 routed experts, top-8 routing.

Recipe (all configs):
  * ``numpy.random.SeedSequence(seed)`` is split into one structure stream
    (offsets, outlier / zero / shift positions) and one value stream per chunk
    of 1024 rows, so the bytes do not depend on the number of threads used;
  * values are drawn in float32 and cast to BF16 with round-to-nearest-even
    (``torch.Tensor.to(torch.bfloat16)`` on the CPU);
  * offsets are ``[0, cumsum(counts)]`` as int32.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

HIDDEN = 7168
INTERMEDIATE = 2048
ROW_CHUNK = 1024


@dataclass
class Segment:
    """One BF16 matrix [M_cap, K] with its expert offsets (length G+1)."""
    name: str
    x_bits: np.ndarray          # uint16 [M_cap, K]
    offs: np.ndarray            # int32 [G+1]

    @property
    def M_cap(self) -> int:
        return int(self.x_bits.shape[0])

    @property
    def K(self) -> int:
        return int(self.x_bits.shape[1])

    @property
    def G(self) -> int:
        return int(self.offs.size - 1)

    @property
    def M_tot(self) -> int:
        return int(self.offs[-1])


@dataclass
class Workload:
    name: str
    description: str
    segments: list[Segment]
    kernels: tuple[str, ...]    # subset of ("quantize", "rows", "cols")
    extra: dict = field(default_factory=dict)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> BF16 bits (uint16) with round-to-nearest-even, via torch CPU."""
    import torch
    x = np.ascontiguousarray(x, dtype=np.float32)
    t = torch.from_numpy(x).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _fill_rows(shape, seeds, draw):
    """Fill a float32 [M, K] array chunk by chunk (1024 rows per child stream)."""
    M, K = shape
    out = np.empty((M, K), np.float32)
    nchunk = (M + ROW_CHUNK - 1) // ROW_CHUNK

    def run(i):
        g = np.random.default_rng(seeds[i])
        r0, r1 = i * ROW_CHUNK, min(M, (i + 1) * ROW_CHUNK)
        out[r0:r1] = draw(g, (r1 - r0, K))

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(run, range(nchunk)))
    return out


def _streams(seed: int, nrows: int, tag: int):
    ss = np.random.SeedSequence([seed, tag])
    nchunk = (nrows + ROW_CHUNK - 1) // ROW_CHUNK
    kids = ss.spawn(1 + nchunk)
    return np.random.default_rng(kids[0]), kids[1:]


def normal(g, shape):
    return g.standard_normal(shape, dtype=np.float32)


def swiglu(g, shape):
    """silu(a) * b with a, b ~ N(0, 1): a SwiGLU intermediate activation."""
    a = g.standard_normal(shape, dtype=np.float32)
    b = g.standard_normal(shape, dtype=np.float32)
    return (a / (1.0 + np.exp(-a))) * b


def student_t3(g, shape):
    return g.standard_t(3.0, shape).astype(np.float32)


def offsets_from_counts(counts) -> np.ndarray:
    counts = np.asarray(counts, dtype=np.int64)
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)


def zipf_weights(n: int, alpha: float, rng) -> np.ndarray:
    w = np.arange(1, n + 1, dtype=np.float64) ** (-alpha)
    return w[rng.permutation(n)]


def avoid_multiples_of_128(counts: np.ndarray) -> np.ndarray:
    """Move one row from any expert whose positive count is a multiple of 128 to
    the next expert, until no positive count is, so every non-empty expert ends in
    a partial tail block."""
    counts = counts.copy()
    G = counts.size
    changed = True
    while changed:
        changed = False
        for g in range(G):
            if counts[g] > 0 and counts[g] % 128 == 0:
                counts[g] -= 1
                counts[(g + 1) % G] += 1
                changed = True
    return counts


# ---- the five workloads --------------------------------------------------------

def config1(seed: int = 0) -> Workload:
    """One expert, 256 x 512: N(0,1), 1% outliers x50, two all-zero 32-blocks."""
    M, K = 256, 512
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K), dtype=np.float32)
    n_out = int(round(0.01 * M * K))
    idx = rng.choice(M * K, n_out, replace=False)
    x.reshape(-1)[idx] *= 50.0
    zb = rng.choice(M * K // 32, 2, replace=False)
    x.reshape(-1, 32)[zb] = 0.0
    seg = Segment("x", to_bf16_bits(x), offsets_from_counts([M]))
    return Workload("config1", "one expert, BF16 256x512, N(0,1) + 1% outliers x50 + two zero 32-blocks",
                    [seg], ("quantize", "rows", "cols"))


def config2(seed: int = 0, rows: int = 32768, K: int = HIDDEN, G: int = 32) -> Workload:
    """MoE dispatch activations: 32768 routed rows (4096 tokens x top-8) over 32
    local experts, counts ~ Multinomial(Dirichlet(0.3)), values N(0,1)."""
    srng, seeds = _streams(seed, rows, 2)
    p = srng.dirichlet(np.full(G, 0.3))
    counts = srng.multinomial(rows, p)
    x = _fill_rows((rows, K), seeds, normal)
    seg = Segment("hidden", to_bf16_bits(x), offsets_from_counts(counts))
    return Workload("config2", f"MoE dispatch, BF16 {rows}x{K}, {G} experts, Dirichlet(0.3) counts, N(0,1)",
                    [seg], ("quantize", "rows"))


def config3(seed: int = 0, rows: int = 32768, K: int = INTERMEDIATE, G: int = 32) -> Workload:
    """Wgrad path: SwiGLU intermediate, ragged Zipf(1.2) counts over 32 experts, no
    non-empty count a multiple of 128 (every expert has a partial tail block)."""
    srng, seeds = _streams(seed, rows, 3)
    w = zipf_weights(G, 1.2, srng)
    counts = srng.multinomial(rows, w / w.sum())
    counts = avoid_multiples_of_128(counts)
    x = _fill_rows((rows, K), seeds, swiglu)
    seg = Segment("intermediate", to_bf16_bits(x), offsets_from_counts(counts))
    return Workload("config3", f"Wgrad, SwiGLU BF16 {rows}x{K}, {G} experts, Zipf(1.2) ragged counts",
                    [seg], ("quantize", "cols"))


def config4(seed: int = 0, rows: int = 65536, K: int = HIDDEN) -> Workload:
    """Dense stress, single segment: Student-t(3) values, 5% zero 32-blocks, 5% of
    blocks with amax set to an exact power of two, 2% of 128-groups with sub-blocks
    1..3 shifted down by 2^-d (d in 9..14), 1% of rows shifted down by 2^-d, 0.1% of
    blocks scaled by 2^-130 (BF16 subnormals)."""
    srng, seeds = _streams(seed, rows, 4)
    x = _fill_rows((rows, K), seeds, student_t3)
    blocks = x.reshape(-1, 32)
    nblk = blocks.shape[0]
    # 5% of 32-blocks zeroed
    zero = srng.random(nblk) < 0.05
    blocks[zero] = 0.0
    # 5% of blocks: the largest element becomes +-2^ceil(log2(amax))
    pw = np.nonzero((srng.random(nblk) < 0.05) & ~zero)[0]
    sub = blocks[pw]
    am = np.argmax(np.abs(sub), axis=1)
    v = sub[np.arange(pw.size), am]
    e = np.ceil(np.log2(np.abs(v).astype(np.float64)))
    blocks[pw, am] = (np.sign(v) * np.exp2(e)).astype(np.float32)
    # 2% of 128-groups: sub-blocks 1..3 scaled by 2^-d, d in 9..14 (row-direction gaps)
    groups = x.reshape(-1, 128)
    gsel = np.nonzero(srng.random(groups.shape[0]) < 0.02)[0]
    gd = srng.integers(9, 15, size=gsel.size)
    groups[gsel, 32:] *= np.exp2(-gd.astype(np.float64)).astype(np.float32)[:, None]
    # 1% of rows scaled by 2^-d (column-direction gaps)
    rsel = np.nonzero(srng.random(rows) < 0.01)[0]
    rd = srng.integers(9, 15, size=rsel.size)
    x[rsel] *= np.exp2(-rd.astype(np.float64)).astype(np.float32)[:, None]
    # 0.1% of blocks scaled by 2^-130: BF16 subnormals, scale byte at its floor
    tsel = np.nonzero(srng.random(nblk) < 0.001)[0]
    blocks[tsel] *= np.float32(2.0 ** -130)
    seg = Segment("dense", to_bf16_bits(x), offsets_from_counts([rows]))
    return Workload("config4", f"dense stress, BF16 {rows}x{K}, Student-t(3), zero / pow2 / shifted / subnormal blocks",
                    [seg], ("quantize", "rows", "cols"))


def config5(seed: int = 0, rows: int = 65536, G: int = 8, experts: int = 256,
            hidden: int = HIDDEN, inter: int = INTERMEDIATE) -> Workload:
    """Full forward chain on one GPU's share of 256 experts (8 local): Zipf(1.2)
    weights over 256 experts under a random permutation, local experts 0..7
    renormalised, multinomial counts, two local experts forced empty (their rows
    go to the largest); hidden 7168 N(0,1) and intermediate 2048 SwiGLU share the
    offsets."""
    srng, seeds_h = _streams(seed, rows, 5)
    _, seeds_i = _streams(seed, rows, 6)
    w = zipf_weights(experts, 1.2, srng)[:G]
    counts = srng.multinomial(rows, w / w.sum())
    empty = srng.choice(G, 2, replace=False)
    moved = int(counts[empty].sum())
    counts[empty] = 0
    counts[int(np.argmax(counts))] += moved
    offs = offsets_from_counts(counts)
    xh = _fill_rows((rows, hidden), seeds_h, normal)
    hs = Segment("hidden", to_bf16_bits(xh), offs)
    del xh
    xi = _fill_rows((rows, inter), seeds_i, swiglu)
    iseg = Segment("intermediate", to_bf16_bits(xi), offs.copy())
    return Workload("config5", f"forward chain, {G} local of {experts} experts, {rows} routed rows, "
                    f"hidden {hidden} N(0,1) + intermediate {inter} SwiGLU",
                    [hs, iseg], ("quantize", "rows", "cols"))


CONFIGS = {1: config1, 2: config2, 3: config3, 4: config4, 5: config5}


def make_config(i: int, seed: int = 0, **kw) -> Workload:
    return CONFIGS[i](seed, **kw)


# ---- small ragged cases for parity tests -----------------------------------------

def ragged_case(counts, K: int, seed: int = 0, values: str = "normal",
                M_cap: int | None = None) -> Segment:
    """A small ragged segment with explicit per-expert counts (empty experts and
    partial tail blocks allowed) and optional capacity slack beyond offs[G]."""
    counts = np.asarray(counts, dtype=np.int64)
    M_tot = int(counts.sum())
    M_cap = M_tot if M_cap is None else M_cap
    assert M_cap >= M_tot
    draw = {"normal": normal, "swiglu": swiglu, "t3": student_t3}[values]
    _, seeds = _streams(seed, max(1, M_cap), 7)
    x = _fill_rows((M_cap, K), seeds, draw) if M_cap > 0 else np.zeros((0, K), np.float32)
    return Segment("ragged", to_bf16_bits(x), offsets_from_counts(counts))
