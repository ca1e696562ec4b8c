// strips.h -- the machinery the transposed-column kernels share: the expert walk over
// 128-row strips of ragged segments, the k-major LDS ring of output columns, the
// monotonic LDS progress counters, and the consumer waves that write each column's
// bytes as whole 128-byte output lines.  Used by cols.hip (MXFP4 -> FP8 columns) and
// fp8q_cols.hip (BF16 -> FP8 columns).
//
// Output layout (technical summary section 2, item 3 of "Practical FP4 Training for
// Large-Scale MoE Models on Hopper GPUs": the Wgrad operand is the per-expert
// transpose, ragged, without padding): expert g's transpose [K, M_g] starts at byte
// K*offs[g], element (k, m') at k*M_g + m'; its block scales [nb_g, K] start at byte
// K*B_g, B_g the number of 128-row blocks of experts 0..g-1 (nb_h = ceil(M_h / 128)).
//
// A strip is one 128-row block of one expert; the strips of all experts are numbered
// in expert order (strip s is row s of the block-scale output).  A workgroup owns a
// 256-column tile and a contiguous range of strips (or every parts-th strip of a segment
// whose strips are independent, kDealRows); its producer waves write each
// strip into the ring and its consumer waves write the strip before to HBM:
// 8 lanes per output column, lane c stores bytes [16c, 16c + 16) of the column's
// 128-byte line, 8 columns per instruction, 32 instructions per strip.  The 8
// columns of an instruction are 16 apart, so their misalignment (mod 16) is the same
// (wave-uniform) and the realignment is five dword LDS reads plus four
// v_alignbyte_b32, with no branch.  A column's stores advance on 128-byte line
// boundaries: the bytes past a strip's last line boundary stay in the ring and go
// out with the next strip, so in the steady state every store covers whole 128-byte
// lines (a partial line costs the memory system a read-modify-write).  Only at the
// ends of a workgroup's run inside an expert are partial lines written.  The output
// is written once and never re-read here, so the stores are streaming.
//
// LDS ring: column k's ring (512 bytes = four strips, with its first 32 bytes repeated
// after it so a 32-byte read window never wraps) starts at byte 544k + 32 (k >> 5), the
// skew against bank conflicts.  Synchronisation is by monotonic counters in LDS (no
// barrier inside the strip loop); every wait is bounded (a wave that waits about a
// second gives up, marks the device's status word and leaves the kernel instead of
// hanging).
#pragma once

#include <atomic>

#include "common.h"

namespace mxfp4 {

constexpr int kStripRows = 128;                      // one FP8 block along the tokens
constexpr int kTileCols = 256;                       // columns of a workgroup's tile
constexpr int kSlots = 4;                            // ring slots (strips) per column
constexpr int kRing = kSlots * kStripRows;           // 512
constexpr int kMirror = 32;                          // ring bytes 0..31 repeated after the ring
constexpr int kColBytes = kRing + kMirror;           // 544
// column k's ring starts at byte 544k + 32 (k >> 5): non-decreasing, so the rings
// never overlap
constexpr int kTileBytes = kTileCols * kColBytes + 32 * ((kTileCols - 1) / 32);

// Values the compiler cannot prove wave-uniform (they come through cross-lane ops or
// LDS) are moved to scalar registers, so branches on them are scalar branches.
__device__ __forceinline__ uint32_t uniform(uint32_t x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int32_t uniform(int32_t x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int64_t uniform(int64_t x)
{
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ uint32_t lds_col(uint32_t kk)
{
    return kColBytes * kk + 32 * (kk >> 5);
}

// ---- strip loads ---------------------------------------------------------------------

// Producers read a strip through a buffer resource whose base is the strip's first row
// and whose range is its rows that exist: a load past the range (a row past a partial
// strip, the last of an expert) returns zero instead of touching memory.  Lane offsets
// within a strip are then the same for every strip (computed once), so a strip's loads
// are issued with no vector arithmetic in front of them; temporaries there make the
// compiler wait for loads still in flight before it reuses their registers, which
// empties the prefetch.
constexpr int kBufferWord3 = 0x00020000;          // gfx9 buffer resource word 3 (32-bit data)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t strip_rsrc(const void* base, uint64_t range)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                             (int)(range > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)range),
                                             kBufferWord3);
}

// ---- progress counters in LDS --------------------------------------------------------

// A wave whose wait ran out of polls sets the device's status word (a vector atomic,
// the same value from every lane) and then leaves the kernel instead of hanging.
__device__ __forceinline__ void give_up(const WaitCtl& w)
{
    __hip_atomic_fetch_or(w.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait (wave-uniformly) until *ctr >= target, at most w.limit polls (false: gave up).
// The acquire orders this wave's later LDS reads after the writes that the counter's
// release published.
__device__ __forceinline__ bool wait_at_least(uint32_t* ctr, uint32_t target, const WaitCtl& w)
{
    for (uint32_t i = 0; i < w.limit; ++i) {
        if (uniform(__hip_atomic_load(ctr, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP)) >= target)
            return true;
        __builtin_amdgcn_s_sleep(1);
    }
    give_up(w);
    return false;
}

// Wait (wave-uniformly) until each of the N counters ctr[0..N-1] is >= target.
template <int N>
__device__ __forceinline__ bool wait_all_at_least(uint32_t* ctr, uint32_t target, const WaitCtl& w)
{
    for (uint32_t i = 0; i < w.limit; ++i) {
        uint32_t m = 0xFFFFFFFFu;
#pragma unroll
        for (int k = 0; k < N; ++k)
            m = min(m, __hip_atomic_load(ctr + k, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP));
        if (uniform(m) >= target)
            return true;
        __builtin_amdgcn_s_sleep(1);
    }
    give_up(w);
    return false;
}

// Count this wave's step as done: the release waits for the wave's own LDS accesses
// (writes it publishes, reads of a slot it frees) before the increment.
__device__ __forceinline__ void signal(uint32_t* ctr)
{
    if ((threadIdx.x & 63) == 0)
        __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// The 16 LDS bytes starting `o` (< 16, the same in every lane) bytes past the 16-byte
// aligned address src: five dwords read from the dword-aligned start, each output dword
// one v_alignbyte_b32 by o & 3 (a shift of zero returns the low dword), with no branch on
// o & 3; the bytes read lie in [src, src + 32).  (An unaligned ds_read_b128 gives the same bytes but measured about
// twelve times slower on MI355X.)
__device__ __forceinline__ u32x4 read_window16(const uint8_t* src, uint32_t o)
{
    // o is wave-uniform: a window that starts on a 16-byte boundary (a column whose
    // output starts on one, as every column of a dealt segment does) is one aligned read
    if (uniform(o) == 0)
        return *reinterpret_cast<const u32x4*>(src);
    const uint32_t* const w = reinterpret_cast<const uint32_t*>(src + (o & ~3u));
    const uint32_t d0 = w[0], d1 = w[1], d2 = w[2], d3 = w[3], d4 = w[4];
    const uint32_t b = o & 3u;
    return u32x4{__builtin_amdgcn_alignbyte(d1, d0, b), __builtin_amdgcn_alignbyte(d2, d1, b),
                 __builtin_amdgcn_alignbyte(d3, d2, b), __builtin_amdgcn_alignbyte(d4, d3, b)};
}

// Bytes [x, y) (0 <= x < y <= 16, not the whole piece) of the 16-byte value v, to
// p + x .. p + y - 1 (p 16-byte aligned), touching no other byte, with naturally aligned
// stores of 1, 2, 4 and 8 bytes.  The partial pieces at a column's ends are a suffix
// [x, 16) or a prefix [0, y): the binary digits of 16 - x (of y) give at most one store
// of each size, so a wave issues four masked stores for all its suffix and prefix
// pieces.  A piece cut on both sides (a column shorter than 16 bytes) grows from x to
// the next boundary and shrinks towards y, at most two stores of each size.
__device__ __forceinline__ void store_part16(uint8_t* p, const u32x4 v, uint32_t x, uint32_t y)
{
    auto dword_at = [&](uint32_t a) {             // the dword holding byte a
        return a < 8 ? (a < 4 ? v.x : v.y) : (a < 12 ? v.z : v.w);
    };
    auto put = [&](uint32_t a, int size) {        // `size` bytes at offset a (a multiple of size)
        if (size == 8) {
            const uint64_t q = a < 8 ? (((uint64_t)v.y << 32) | v.x) : (((uint64_t)v.w << 32) | v.z);
            __builtin_nontemporal_store(q, reinterpret_cast<uint64_t*>(p + a));
        } else if (size == 4) {
            __builtin_nontemporal_store(dword_at(a), reinterpret_cast<uint32_t*>(p + a));
        } else if (size == 2) {
            __builtin_nontemporal_store((uint16_t)(dword_at(a) >> (8 * (a & 3))), reinterpret_cast<uint16_t*>(p + a));
        } else {
            __builtin_nontemporal_store((uint8_t)(dword_at(a) >> (8 * (a & 3))), p + a);
        }
    };
    if (x > 0 && y < 16) {
        uint32_t a = x;
#pragma unroll
        for (int size = 1; size <= 8; size <<= 1)
            if ((a & (uint32_t)size) && a + size <= y) {
                put(a, size);
                a += size;
            }
#pragma unroll
        for (int size = 8; size >= 1; size >>= 1)
            if (a + size <= y) {
                put(a, size);
                a += size;
            }
        return;
    }
    const bool suffix = x > 0;
#pragma unroll
    for (int size = 1; size <= 8; size <<= 1) {
        const uint32_t s = (uint32_t)size;
        // suffix: x rounded up to a multiple of the size; prefix: y's bits above the size
        const bool has = suffix ? ((16u - x) & s) != 0 : (y & s) != 0;
        const uint32_t at = suffix ? (x + s - 1) & ~(s - 1) : y & ~(2 * s - 1);
        if (has)
            put(at, size);
    }
}

// ---- strips of experts ----------------------------------------------------------------

// Per-lane expert table for experts g0 + lane: first strip, strip count, first row and
// row count.  Every wave builds it on its own (no barrier).
struct ExpertTable {
    uint32_t sb, ns;           // first strip, strip count (lane's expert)
    int32_t row0, mg;          // first row, rows
    uint32_t total;            // strips of the whole chunk
};

__device__ __forceinline__ ExpertTable expert_chunk(const int32_t* __restrict__ offs, int G, int g0,
                                                    uint32_t run)
{
    const int lane = threadIdx.x & 63;
    const int h = g0 + lane;
    ExpertTable t;
    t.row0 = h < G ? offs[h] : 0;
    t.mg = h < G ? offs[h + 1] - t.row0 : 0;
    t.ns = (uint32_t)(t.mg + kStripRows - 1) / kStripRows;
    uint32_t incl = t.ns;
#pragma unroll
    for (int dlt = 1; dlt < 64; dlt <<= 1) {
        uint32_t other = __shfl_up(incl, dlt, 64);
        if (lane >= dlt)
            incl += other;
    }
    t.sb = run + incl - t.ns;
    t.total = uniform((uint32_t)__shfl(incl, 63, 64));
    return t;
}

struct StripInfo {
    int64_t row0, mg;          // expert's first row and row count
    uint32_t g;                // expert
    uint32_t sb, ns;           // expert's first strip and strip count
    uint32_t s;                // this strip (= its row in the block-scale output)
    int64_t r_lo;              // the strip's first row, relative to row0
    int nrows;                 // rows in the strip
};

__device__ __forceinline__ void set_rows(StripInfo& r)
{
    r.r_lo = (int64_t)(r.s - r.sb) * kStripRows;
    r.nrows = (int)min<int64_t>(kStripRows, r.mg - r.r_lo);
}

// Expert of global strip s (s < total strips), searched 64 experts at a time with
// one lane per expert.  `cached` is the table of experts 0..63.  Used once per
// workgroup, before the strip loop.
__device__ __forceinline__ StripInfo locate(const int32_t* __restrict__ offs, int G,
                                            const ExpertTable& cached, uint32_t s)
{
    ExpertTable t = cached;
    uint32_t run = 0;
    for (int g0 = 0;; g0 += 64) {
        if (g0 > 0)
            t = expert_chunk(offs, G, g0, run);
        const bool mine = t.ns > 0 && s >= t.sb && s < t.sb + t.ns;
        const uint64_t mask = __ballot(mine);
        if (mask || g0 + 64 >= G) {
            const int src = mask ? __builtin_ctzll(mask) : 0;
            StripInfo r;
            r.row0 = uniform((int32_t)__builtin_amdgcn_readlane(t.row0, src));
            r.mg = uniform((int32_t)__builtin_amdgcn_readlane(t.mg, src));
            r.sb = uniform((uint32_t)__builtin_amdgcn_readlane(t.sb, src));
            r.ns = uniform((uint32_t)__builtin_amdgcn_readlane(t.ns, src));
            r.g = (uint32_t)(g0 + src);
            r.s = s;
            set_rows(r);
            return r;
        }
        run += t.total;
    }
}

// Strip p.s + step (which exists).  Inside the strip loop the experts are walked one
// by one with scalar loads of the offsets (counted apart from the vector loads, so
// the prefetched rows are never waited for early).
__device__ __forceinline__ StripInfo next_strip(const int32_t* __restrict__ offs, int G,
                                                const StripInfo& p, uint32_t step = 1)
{
    StripInfo r = p;
    r.s = p.s + step;
    while (r.s >= r.sb + r.ns && (int)r.g + 1 < G) {
        r.sb += r.ns;
        int64_t end = r.row0 + r.mg;
        uint32_t g = r.g;
        do {                                   // skip empty experts
            ++g;
            r.row0 = end;
            end = offs[g + 1];
        } while (end == r.row0 && (int)g + 1 < G);
        r.g = g;
        r.mg = end - r.row0;
        r.ns = (uint32_t)((r.mg + kStripRows - 1) / kStripRows);
    }
    set_rows(r);
    return r;
}

// Experts whose row counts are all multiples of this many rows make every strip of the
// segment independent: each column of each expert then starts on a 128-byte output
// line (K, the expert's first row and the column length M_g are multiples of 128), so
// no strip carries bytes into the next and any strip can be written alone.  The column
// kernels then deal a tile's strips to its workgroups in turn (workgroup `part` takes
// strips part, part + parts, ...): at any time the workgroups of a tile write
// neighbouring lines of every column, instead of lines one contiguous range apart.
// With a column length that is a multiple of a large power of two the contiguous
// ranges put the concurrent lines of all columns at one address modulo that power;
// dealt strips ran 7-15 % faster in memory-only probes of that traffic on MI355X
// (65536-row columns), and about the same (within a few per cent either way) with
// column lengths that are multiples of 128 only, so they are used from 4096 rows up.
constexpr int kDealRows = 4096;

// Strips of all experts and whether every expert's row count is a multiple of
// kDealRows (an empty expert is).  `t0` is the table of experts 0..63.
struct SegmentScan {
    uint32_t n_strips;
    bool dealt;
};

__device__ __forceinline__ SegmentScan scan_segment(const int32_t* __restrict__ offs, int G,
                                                    const ExpertTable& t0)
{
    SegmentScan r;
    r.n_strips = t0.total;
    bool dealt = __ballot((t0.mg & (kDealRows - 1)) != 0) == 0;
    for (int g0 = 64; g0 < G; g0 += 64) {
        const ExpertTable t = expert_chunk(offs, G, g0, r.n_strips);
        r.n_strips = uniform(r.n_strips + t.total);
        dealt = dealt && __ballot((t.mg & (kDealRows - 1)) != 0) == 0;
    }
    r.dealt = dealt;
    return r;
}

// This workgroup's strips: first strip, stride between its strips and how many it
// converts (a lead-in strip included).  Contiguous ranges [s0, s1) of the segment's
// strips split over `parts` workgroups per tile, except for a dealt segment
// (kDealRows); false if the workgroup has none.  A range that starts inside an expert
// also converts the strip before it (a lead-in strip that writes nothing): its bytes
// past its last line boundary complete the first output line of the range, so the
// workgroup writes that line whole and the workgroup before it stops at its last line
// boundary (lines split between two workgroups would otherwise be written partially
// twice).  An expert whose row count is a multiple of 128 needs none: every strip of it
// starts and ends on a line boundary of every column, so nothing is carried.
struct StripRun {
    StripInfo first;           // first strip converted (the lead-in strip, if any)
    uint32_t step;             // strips from one to the next
    uint32_t n;                // strips converted
    bool lead;                 // the first strip is a lead-in strip
    bool dealt;                // independent strips: none continues another
};

__device__ __forceinline__ bool strip_run(const int32_t* __restrict__ offs, int G, const ExpertTable& t0,
                                          uint32_t part, uint32_t parts, StripRun& run)
{
    const SegmentScan sc = scan_segment(offs, G, t0);
    run.dealt = sc.dealt;
    if (sc.dealt) {
        if (part >= sc.n_strips)
            return false;
        run.first = locate(offs, G, t0, part);
        run.step = parts;
        run.n = (sc.n_strips - part + parts - 1) / parts;
        run.lead = false;
        return true;
    }
    const uint32_t s0 = (uint32_t)(((uint64_t)sc.n_strips * part) / parts);
    const uint32_t s1 = (uint32_t)(((uint64_t)sc.n_strips * (part + 1)) / parts);
    if (s0 >= s1)
        return false;
    StripInfo f = locate(offs, G, t0, s0);
    run.lead = f.s > f.sb && (f.mg & (kStripRows - 1)) != 0;
    if (run.lead) {
        f.s -= 1;
        set_rows(f);
    }
    run.first = f;
    run.step = 1;
    run.n = s1 - s0 + (run.lead ? 1u : 0u);
    return true;
}

// What the producers hand to the consumers for one ring slot.
struct SlotInfo {
    int64_t A0;                // output byte of (tile column 0, strip row 0)
    int32_t mg;                // rows of the expert (= output row length)
    int32_t nrows;             // rows in the strip
    uint32_t blk;              // row of the block-scale output
    uint32_t flags;            // bit 0: the ring holds the previous strip of the same expert;
                               // bit 1: the next strip (of the whole numbering) is of the
                               // same expert; bit 2: lead-in strip (write nothing)
    uint32_t S[2];             // block scale byte of MX groups 0..7 of the tile
};

// ---- consumers ---------------------------------------------------------------------------

// A consumer lane writes one aligned 16-byte chunk of one column per strip: lane
// (mc = lane >> 3, c = lane & 7) of store instruction g (0..31) of the strip owns tile
// column kk = 2 (g >> 2) + ((g & 3) >> 1) + 16 mc + 128 (g & 1) and bytes [16c, 16c + 16)
// of the column's 128-byte output line, so the 8 lanes of a column store one whole line.
// Within a run of strips of one expert the column's line phase is fixed, so this
// state is set at the first strip and advanced by 128 bytes per strip.
template <int N>
struct ColState {
    uint32_t q[N];             // ring offset of the lane's chunk, minus the strip's slot base
    uint8_t* p[N];             // output address of the lane's chunk
    uint32_t o[N];             // misalignment (wave-uniform): (-A) & 15
};

// The consumer waves' loop, shared by the column kernels: wave v (0 .. kConsumerWaves - 1
// of the consumers) writes store instructions v, v + kConsumerWaves, ... (< 32) of every
// strip the workgroup converts, once wait_produced(t) has seen every producer wave
// finish strip t (false: the wait gave up, leave), and counts the slot in
// `drained[slot]` when done.  Consumer wave 0 also calls write_scales(slot) for every
// strip that is not a lead-in strip.
template <int kConsumerWaves, typename WaitProduced, typename WriteScales>
__device__ __forceinline__ void consume_strips(uint8_t* tile, const SlotInfo* info, uint32_t* drained,
                                               uint8_t* __restrict__ yT, int ncols, uint32_t n, int v,
                                               WaitProduced wait_produced, WriteScales write_scales)
{
    constexpr int kMaxIts = (32 + kConsumerWaves - 1) / kConsumerWaves;
    const int lane = threadIdx.x & 63;
    const int mc = lane >> 3;
    const int c = lane & 7;                       // bytes [16c, 16c + 16) of the line
    // store instruction k of this wave is instruction g = v + kConsumerWaves k (< 32) of the
    // strip: tile columns 2 (g >> 2) + ((g & 3) >> 1) + 16 mc + 128 (g & 1)
    auto col_of = [&](int g) { return (uint32_t)(2 * (g >> 2) + ((g & 3) >> 1) + 16 * mc + 128 * (g & 1)); };
    ColState<kMaxIts> cs;
    for (uint32_t t = 0; t < n; ++t) {
        if (!wait_produced(t))
            return;
        const uint32_t slot = t % kSlots;
        const int64_t A0 = uniform(info[slot].A0);
        const int64_t mg = uniform(info[slot].mg);
        const int64_t nrows = uniform(info[slot].nrows);
        const uint32_t flags = uniform(info[slot].flags);
        const bool cin = flags & 1u, cout = flags & 2u, skip = flags & 4u;
        const uint32_t slot_base = kStripRows * slot;

        if (!skip && v == 0)
            write_scales(slot);
        if (!cin) {
#pragma unroll
            for (int k = 0; k < kMaxIts; ++k) {
                const int g = v + kConsumerWaves * k;
                if (g >= 32)
                    continue;
                const uint32_t kk = col_of(g);
                const int64_t A = A0 + (int64_t)kk * mg;
                const uint32_t a = (uint32_t)A & 127;
                cs.o[k] = uniform((uint32_t)(16 - (A & 15)) & 15);
                cs.q[k] = 16 * c - a - cs.o[k];
                cs.p[k] = yT + (A - a) + 16 * c;
            }
        }
        if (skip) {
#pragma unroll
            for (int k = 0; k < kMaxIts; ++k)
                cs.p[k] += kStripRows;
        } else if (cin && cout) {
#pragma unroll
            for (int k = 0; k < kMaxIts; ++k) {
                const int g = v + kConsumerWaves * k;
                if (g >= 32 || ((g & 1) && ncols <= 128))
                    continue;
                const uint8_t* const src = tile + lds_col(col_of(g)) + ((cs.q[k] + slot_base) & (kRing - 1));
                store_stream(reinterpret_cast<u32x4*>(cs.p[k]), read_window16(src, cs.o[k]));
                cs.p[k] += kStripRows;
            }
        } else {
#pragma unroll
            for (int k = 0; k < kMaxIts; ++k) {
                const int g = v + kConsumerWaves * k;
                if (g >= 32 || ((g & 1) && ncols <= 128))
                    continue;
                const uint32_t kk = col_of(g);
                const int64_t A = A0 + (int64_t)kk * mg;
                const uint32_t o = cs.o[k];
                const int64_t E = A + nrows;
                const int64_t W_lo = cin ? (A & ~(int64_t)127) : A;
                const int64_t W_hi = cout ? (E & ~(int64_t)127) : E;
                const int64_t j0 = W_lo >> 4;
                const int nch = W_hi > W_lo ? (int)(((W_hi + 15) >> 4) - j0) : 0;
                const uint8_t* const colp = tile + lds_col(kk);
                for (int pass = 0; pass < 2; ++pass) {
                    const int jj = c + 8 * pass;
                    if (jj >= nch)
                        continue;
                    const int64_t b0 = (j0 + jj) << 4;
                    const uint32_t pos = (slot_base + (uint32_t)(b0 - A) - o) & (kRing - 1);
                    const u32x4 val = read_window16(colp + pos, o);
                    if (b0 >= W_lo && b0 + 16 <= W_hi) {
                        store_stream(reinterpret_cast<u32x4*>(yT + b0), val);
                    } else {
                        store_part16(yT + b0, val, (uint32_t)max<int64_t>(W_lo - b0, 0),
                                     (uint32_t)min<int64_t>(W_hi - b0, 16));
                    }
                }
                cs.p[k] += kStripRows;
            }
        }
        signal(&drained[slot]);
    }
}

// Compute units of the current device, read once per device.  Concurrent first calls
// may both read the attribute; they store the same value.
static inline int device_cus()
{
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

}  // namespace mxfp4
