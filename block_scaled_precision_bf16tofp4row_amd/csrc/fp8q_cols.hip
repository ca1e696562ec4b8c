// fp8q_cols.hip -- the backward FP8 quantizer in transposed column layout (WGRAD
// operand): BF16 -> FP8 E4M3FN with one UE8M0 scale per 1x128 block along the tokens
// of each expert, over ragged per-expert segments, transpose fused.
//
// Method: "Practical FP4 Training for Large-Scale MoE Models on Hopper GPUs",
// technical summary section 2: the backward pass (item 2) keeps gradients on the
// standard FP8 path, E4M3 with 128-element blocks (item 1); the Wgrad operand is the
// per-expert transpose over ragged segments without padding (item 3).  Scale rule
// and element rounding are those of the row quantizer (fp8q.hip): for each 128-row
// block b of an expert and each column k, S = floor(log2 amax) - 8 + 127 clamped to
// [0, 254] over the rows of the block that exist, elements x / 2^(S-127) rounded to
// nearest even, saturating at +-448, sign kept.  Output layout and the ring /
// consumer machinery are those of strips.h (same layout as the MXFP4 -> FP8 column
// conversion).
//
// Producers (waves 0-7): wave w = 4b + q quantizes the 128 columns of block b (tile
// columns 128b .. 128b + 127) over rows 32q..32q+31 of every strip.  Lane (c = lane & 15,
// rg = lane >> 4) holds rows 32q + 8rg .. + 7 of columns 128b + 8c .. + 7 (one 16-byte
// chunk per row; the lanes of a load instruction read 4 rows x 256 bytes).  Loads run
// kQPrefetch strips ahead.  A column's amax is reduced over the lane's eight rows
// (packed 16-bit max on the magnitude bits) and the wave's four row groups (the gfx950
// 16- and 32-lane swaps), published to a per-slot LDS array, and combined with the
// other three waves of the block once they have published theirs (bounded waits on
// per-wave counters); the two blocks run independently, so the consumers wait for every
// producer wave's own counter.  (A layout in which each wave held 32 columns over all
// 128 rows needs no exchange, but its load instructions read 16 rows x 64 bytes: 1.5-2.4 %
// slower for the column layout alone, and 10-14 % slower with the row layout below,
// whose rows it splits over four waves.)
// The element convert, v_cvt_scalef32_pk_fp8_bf16, takes one scale for a pair of
// BF16, and neighbouring columns have different scales, so a pair is two rows of one
// column (one v_perm_b32): the four converts of a column's eight rows give its eight
// ring bytes, rows in order, with no byte transpose.  As in the row quantizer,
// magnitudes are clamped to 448 * 2^(S-127) before the convert (it returns NaN for
// quotients of 464 or more instead of saturating).
// Consumers (waves 8-15): strips.h.
//
// With kRows the kernel also writes the row layout of the same gradient (DGRAD operand,
// 1x128 blocks along K, the row quantizer's output) from the same read.  A row's
// 128-column block is one wave's, so its maximum needs no exchange (the sixteen lanes of
// a row group, two DPP quad permutes and two row rotations) and its 128 FP8 bytes go out
// as one whole line; the wave stores its rows and the scale bytes through resources over
// the strip's rows.  Loop-invariant offsets are then recomputed from an opaque lane
// index each strip, because holding them spills, and a spill reload in the loop would
// wait for the prefetched strip.
#include "strips.h"

namespace mxfp4 {

typedef __bf16 qbf16x2 __attribute__((ext_vector_type(2)));

constexpr int kQProducerWaves = 8;                          // 128 columns x 32 rows each
constexpr int kQConsumerWaves = 8;
constexpr int kQPrefetch = 1;                               // strips of loads in flight
constexpr int kQThreads = 64 * (kQProducerWaves + kQConsumerWaves);
static_assert(kTileCols == 32 * kQProducerWaves, "a producer wave quantizes 32 columns");
static_assert(kStripRows == 128, "sixteen row groups of eight rows");
static_assert((kRing & (kRing - 1)) == 0, "the ring position wraps with a mask");

namespace {

// A lane's eight rows of a strip: v[i] holds 8 BF16 (columns 128b + 8c .. + 7) of row
// 32q + 8rg + i.
struct QRows {
    u32x4 v[8];
};

// Loads go through strip_rsrc (strips.h): rows past a partial strip read as zero, which
// leaves the column amax unchanged; their converted bytes are never written out.  The
// lane's byte offsets (row * 2K + column byte) fit in 32 bits (128 rows x 2K bytes with
// K <= 2^24; the range is capped at 2^32 - 1, far above the last valid offset).
__device__ __forceinline__ QRows load_rows(const uint8_t* __restrict__ x, int64_t K, const StripInfo& st,
                                           uint32_t kt, const uint32_t (&off)[8])
{
    QRows in;
    const __amdgpu_buffer_rsrc_t rsrc = strip_rsrc(x + (st.row0 + st.r_lo) * (2 * K) + 512 * (int64_t)kt,
                                                   (uint64_t)st.nrows * (uint64_t)(2 * K));
#pragma unroll
    for (int i = 0; i < 8; ++i)
        in.v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)off[i], 0, 0));
    return in;
}

__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b)
{
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                  __builtin_bit_cast(u16x2, b)));
}

__device__ __forceinline__ qbf16x2 as_qbf16x2(uint32_t u)
{
    qbf16x2 r;
    __builtin_memcpy(&r, &u, sizeof(r));
    return r;
}

// Two BF16 of one column (one dword) with that column's clamp pattern and scale ->
// two E4M3FN bytes in half kHi of acc.
template <bool kHi>
__device__ __forceinline__ u16x2 cvt_pair(u16x2 acc, uint32_t w, uint32_t clamp2, float scale)
{
    const uint32_t mag = __builtin_bit_cast(uint32_t, __builtin_elementwise_min(
        __builtin_bit_cast(u16x2, w & 0x7FFF7FFFu), __builtin_bit_cast(u16x2, clamp2)));
    const uint32_t c = mag | (w & 0x80008000u);
    typedef short s16x2_t __attribute__((ext_vector_type(2)));
    const s16x2_t r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(__builtin_bit_cast(s16x2_t, acc),
                                                                as_qbf16x2(c), scale, kHi);
    return __builtin_bit_cast(u16x2, r);
}

}  // namespace

// kRows: also write the row layout (1 x 128 blocks along K) from the same read of x.
template <bool kRows>
__global__ __launch_bounds__(kQThreads, 1) void fp8q_cols_kernel(
    const uint8_t* __restrict__ x, uint8_t* __restrict__ yT, uint8_t* __restrict__ yT_scales,
    uint8_t* __restrict__ y, uint8_t* __restrict__ y_scales, const int32_t* __restrict__ offs, int G,
    int64_t K, int parts, WaitCtl wc)
{
    __shared__ __attribute__((aligned(16))) uint8_t tile[kTileBytes];
    __shared__ __attribute__((aligned(16))) SlotInfo info[kSlots];
    // per ring slot: the block scale byte of each tile column
    __shared__ __attribute__((aligned(16))) uint8_t sbytes[kSlots][kTileCols];
    // strips finished, one counter per producer wave (the producer waves do not run in
    // lockstep, so a summed count would not show that all of them wrote strip t), and
    // per ring slot the strips drained by the consumer waves (all monotonic)
    __shared__ __attribute__((aligned(16))) uint32_t produced[kQProducerWaves];
    __shared__ uint32_t drained[kSlots];
    // per ring slot, each producer wave's maximum magnitude (BF16 bits) of each of its
    // block's 128 columns over its 32 rows, and per wave the strips so published
    __shared__ __attribute__((aligned(16))) uint16_t pmax[kSlots][kQProducerWaves][128];
    __shared__ __attribute__((aligned(16))) uint32_t colpub[kQProducerWaves];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t nkt = (uint32_t)((K + kTileCols - 1) / kTileCols);
    const uint32_t lambda = xcd_remap(blockIdx.x, gridDim.x);
    const uint32_t kt = lambda % nkt;
    const uint32_t part = lambda / nkt;
    const int ncols = (int)min<int64_t>(kTileCols, K - (int64_t)kTileCols * kt);

    // this workgroup's strips of column tile kt (strip_run, strips.h): a contiguous range,
    // with a lead-in strip where it starts inside an expert, or every parts-th strip of
    // a segment whose strips are independent
    const ExpertTable t0 = expert_chunk(offs, G, 0, 0);
    StripRun run;
    if (!strip_run(offs, G, t0, part, (uint32_t)parts, run))
        return;                                   // uniform over the workgroup
    const uint32_t n = run.n;

    if (tid == 0) {
        for (int k = 0; k < kQProducerWaves; ++k) {
            produced[k] = 0;
            colpub[k] = 0;
        }
        for (int k = 0; k < kSlots; ++k)
            drained[k] = 0;
    }
    __syncthreads();                              // the only barrier: counters set

    if (wave < kQProducerWaves) {
        // ================= producers =================
        // wave w = 4b + q quantizes the 128 columns of block b over rows 32q..32q+31; lane
        // (c = lane & 15, rg = lane >> 4) holds rows 32q + 8rg .. + 7 of columns
        // 128b + 8c .. + 7.  The narrow last tile (128 columns) has block 0 only: waves 4-7
        // load its columns again (their ring columns are never written out).
        const int c = lane & 15;
        const int rg = lane >> 4;
        const int blk = wave >> 2;                // the wave's 128-column block
        const int row_g = 32 * (wave & 3) + 8 * rg;   // first of the lane's eight rows
        // first tile column of the lane's eight in a row of x
                const uint32_t ldcol = (ncols > 128 ? (uint32_t)blk : 0u) * 128u + 8u * (uint32_t)c;
        uint32_t off[8];                          // byte offsets of the lane's rows in a strip
#pragma unroll
        for (int i = 0; i < 8; ++i)
            off[i] = (uint32_t)(row_g + i) * (uint32_t)(2 * K) + 2 * ldcol;
        // tile column 128b + 8c + j sits at LDS byte lds_col(128b + 8c) + 544 j

        // column maxima: this wave's maximum of each of the lane's eight
        // columns over its 32 rows (the four row groups of a column are lanes c, c + 16,
        // c + 32, c + 48: the gfx950 16- and 32-lane swaps), published for the other three
        // waves of the block; the block's four are combined once all have published
        auto publish_col_max = [&](const QRows& in, uint32_t slot) {
            uint32_t M[4];
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                uint32_t m = in.v[0][d] & 0x7FFF7FFFu;
#pragma unroll
                for (int i = 1; i < 8; ++i)
                    m = pk_max_u16(m, in.v[i][d] & 0x7FFF7FFFu);
                const auto a = __builtin_amdgcn_permlane16_swap(m, m, false, false);
                m = pk_max_u16(a[0], a[1]);
                const auto b = __builtin_amdgcn_permlane32_swap(m, m, false, false);
                M[d] = pk_max_u16(b[0], b[1]);
            }
            uint32_t ln = (uint32_t)lane;            // opaque, as in produce_rows
            asm volatile("" : "+v"(ln));
            if ((ln >> 4) == 0)
                *reinterpret_cast<u32x4*>(&pmax[slot][wave][8 * (ln & 15)]) = u32x4{M[0], M[1], M[2], M[3]};
        };
        // row layout (no exchange: the row's 128-column block is the wave's): the
        // block scale of each of the lane's rows (the sixteen lanes of a row group hold its
        // 128 columns), its eight bytes of each row and, from lane c = 0, the scale byte.
        // Stores go through resources over the strip's rows, empty for a lead-in strip and
        // for the repeated columns of a narrow tile, so nothing else is written.
        auto produce_rows = [&](const StripInfo& st, const QRows& in, uint32_t flags) {
            // lane-dependent offsets are derived from a lane index the compiler cannot
            // see through (the empty asm), so that it recomputes them here instead of
            // holding them in registers of their own across the strip loop (which spills)
            uint32_t ln = (uint32_t)lane;
            asm volatile("" : "+v"(ln));
            const uint32_t lc = ln & 15, lrow = 32 * (uint32_t)(wave & 3) + 8 * (ln >> 4);
            const bool writes = (flags & 4u) == 0 && (ncols > 128 || wave < 4);
            const int64_t r0 = st.row0 + st.r_lo;
            const uint32_t nr = writes ? (uint32_t)st.nrows : 0u;
            const __amdgpu_buffer_rsrc_t ry = strip_rsrc(y + r0 * K, (uint64_t)nr * (uint64_t)K);
            const __amdgpu_buffer_rsrc_t rs = strip_rsrc(y_scales + r0 * (K / 128), (uint64_t)nr * (uint64_t)(K / 128));
            // byte offsets of the lane's first row
            const uint32_t vrow = lrow * (uint32_t)K + (uint32_t)(kTileCols * kt) + 128 * (uint32_t)blk + 8 * lc;
            const uint32_t vscl = lrow * (uint32_t)(K / 128) + (uint32_t)(2 * kt) + (uint32_t)blk;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                uint32_t m = pk_max_u16(pk_max_u16(in.v[i][0] & 0x7FFF7FFFu, in.v[i][1] & 0x7FFF7FFFu),
                                        pk_max_u16(in.v[i][2] & 0x7FFF7FFFu, in.v[i][3] & 0x7FFF7FFFu));
                m = max(m & 0xFFFFu, m >> 16);
                m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
                m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
                m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x124, 0xF, 0xF, false));  // row_ror:4
                m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x128, 0xF, 0xF, false));  // row_ror:8
                const uint32_t S = (m >> 7) > 8 ? (m >> 7) - 8 : 0u;
                const uint32_t clamp2 = (((S + 8) << 7) | 0x60u) * 0x00010001u;
                const float scale = __uint_as_float(max(S << 23, 0x00400000u));   // S = 0: 2^-127
                u16x2 lo = {0, 0}, hi = {0, 0};
                lo = cvt_pair<false>(lo, in.v[i][0], clamp2, scale);
                lo = cvt_pair<true>(lo, in.v[i][1], clamp2, scale);
                hi = cvt_pair<false>(hi, in.v[i][2], clamp2, scale);
                hi = cvt_pair<true>(hi, in.v[i][3], clamp2, scale);
                __builtin_amdgcn_raw_buffer_store_b64(
                    u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)}, ry,
                    (int)(vrow + (uint32_t)i * (uint32_t)K), 0, 0);
                if (lc == 0)
                    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)S, rs, (int)(vscl + (uint32_t)i * (uint32_t)(K / 128)), 0,
                                                         0);
            }
        };

        auto produce = [&](const StripInfo& st, const QRows& in, uint32_t slot, uint32_t flags) {
            // column maxima over the strip (pairs of columns 128b + 8c + 2d and + 1): the
            // block's four published partial maxima
            uint32_t M[4];
            {
                const int wb = wave & ~3;
                uint32_t ln = (uint32_t)lane;
                asm volatile("" : "+v"(ln));
                const uint32_t pc = 8 * (ln & 15);
                const u32x4 p0 = *reinterpret_cast<const u32x4*>(&pmax[slot][wb + 0][pc]);
                const u32x4 p1 = *reinterpret_cast<const u32x4*>(&pmax[slot][wb + 1][pc]);
                const u32x4 p2 = *reinterpret_cast<const u32x4*>(&pmax[slot][wb + 2][pc]);
                const u32x4 p3 = *reinterpret_cast<const u32x4*>(&pmax[slot][wb + 3][pc]);
                M[0] = pk_max_u16(pk_max_u16(p0.x, p1.x), pk_max_u16(p2.x, p3.x));
                M[1] = pk_max_u16(pk_max_u16(p0.y, p1.y), pk_max_u16(p2.y, p3.y));
                M[2] = pk_max_u16(pk_max_u16(p0.z, p1.z), pk_max_u16(p2.z, p3.z));
                M[3] = pk_max_u16(pk_max_u16(p0.w, p1.w), pk_max_u16(p2.w, p3.w));
            }
            // scale bytes: biased exponent field of the column max minus 8, at least 0
            uint32_t S2[4];               // S of columns 2d (low half) and 2d + 1 (high half)
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const u16x2 e = __builtin_bit_cast(u16x2, M[d]) >> (unsigned short)7;
                const u16x2 eight = {8, 8};
                S2[d] = __builtin_bit_cast(uint32_t, __builtin_elementwise_sub_sat(e, eight));
            }
            // with the row layout there are not enough registers to keep these offsets
            // across the strip loop: derive them from an opaque lane index (see
            // produce_rows)
            uint32_t ln = (uint32_t)lane;
            if constexpr (kRows)
                asm volatile("" : "+v"(ln));
            const uint32_t lrg = ln >> 4, lcc = ln & 15;
            const uint32_t lcol0 = 128 * (uint32_t)blk + 8 * lcc;
            // the block scale bytes, once per tile column: by the lanes holding a column's
            // first row group in the block's first wave
            if (lrg == 0 && (wave & 3) == 0)
                *reinterpret_cast<u32x2*>(&sbytes[slot][lcol0]) =
                    u32x2{perm(S2[1], S2[0], 0x06040200u), perm(S2[3], S2[2], 0x06040200u)};
            if (wave == 0 && lane == 0) {
                info[slot].A0 = K * st.row0 + st.r_lo + (int64_t)kTileCols * kt * st.mg;
                info[slot].mg = (int32_t)st.mg;
                info[slot].nrows = st.nrows;
                info[slot].blk = st.s;
                info[slot].flags = flags;
            }
            // quantize column by column: rows (0, 1), (2, 3), (4, 5), (6, 7) form the
            // four pairs; the two result dwords are the column's eight ring bytes
            const uint32_t lrow = 32 * (uint32_t)(wave & 3) + 8 * lrg;
            uint8_t* const w = tile + lds_col(lcol0) + lrow + kStripRows * slot;
            u32x2 T[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t S = (S2[j >> 1] >> (16 * (j & 1))) & 0xFFu;
                const uint32_t clamp = ((S + 8) << 7) | 0x60u;
                const uint32_t clamp2 = clamp * 0x00010001u;
                const float scale = __uint_as_float(max(S << 23, 0x00400000u));   // S = 0: 2^-127
                const int d = j >> 1;
                const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
                u16x2 lo = {0, 0}, hi = {0, 0};
                lo = cvt_pair<false>(lo, perm(in.v[1][d], in.v[0][d], sel), clamp2, scale);
                lo = cvt_pair<true>(lo, perm(in.v[3][d], in.v[2][d], sel), clamp2, scale);
                hi = cvt_pair<false>(hi, perm(in.v[5][d], in.v[4][d], sel), clamp2, scale);
                hi = cvt_pair<true>(hi, perm(in.v[7][d], in.v[6][d], sel), clamp2, scale);
                T[j] = u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
                *reinterpret_cast<u32x2*>(w + kColBytes * j) = T[j];
            }
            // ring bytes 0..31 (rows 0..31 of slot 0) are repeated after the ring, so a
            // 32-byte read window never wraps
            if (slot == 0 && lrow < 32) {
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    *reinterpret_cast<u32x2*>(w + kRing + kColBytes * j) = T[j];
            }
        };
        // a dealt strip neither continues the ring's previous strip nor carries into the next
        auto flags_of = [&](uint32_t prev_sb, const StripInfo& cur, bool lead_in) {
            if (run.dealt)
                return 0u;
            return (prev_sb == cur.sb ? 1u : 0u) | (cur.s + 1 < cur.sb + cur.ns ? 2u : 0u) | (lead_in ? 4u : 0u);
        };

        // Step t waits until the consumers have drained strip t - 3 (whose slot carries
        // into strip t - 2, the last reader of slot t % 4), quantizes strip t and
        // signals it.  Loads run kQPrefetch strips ahead; register sets rotate over
        // kQPrefetch + 1 strips and the loop is unrolled by that much so each set keeps
        // fixed registers.
        constexpr int kSets = kQPrefetch + 1;
        uint32_t prev_sb = 0xFFFFFFFFu;
        StripInfo I[kSets];
        QRows R[kSets];
        I[0] = run.first;
#pragma unroll
        for (int u = 1; u < kQPrefetch; ++u)
            I[u] = (uint32_t)u < n ? next_strip(offs, G, I[u - 1], run.step) : I[u - 1];
#pragma unroll
        for (int u = 0; u < kQPrefetch; ++u)
            R[u] = load_rows(x, K, I[u], kt, off);
        for (uint32_t t = 0;; t += kSets) {
#pragma unroll
            for (int u = 0; u < kSets; ++u) {
                const uint32_t tt = t + u;
                const int ld = (u + kQPrefetch) % kSets;          // set receiving strip tt + kQPrefetch
                const int pv = (u + kQPrefetch - 1) % kSets;      // set of strip tt + kQPrefetch - 1
                I[ld] = tt + kQPrefetch < n ? next_strip(offs, G, I[pv], run.step) : I[pv];
                if constexpr (kRows) {
                    // not enough registers to keep the eight row offsets across the loop:
                    // recompute them from an opaque lane index (see produce_rows)
                    uint32_t ln = (uint32_t)lane;
                    asm volatile("" : "+v"(ln));
                    const uint32_t lcol = (ncols > 128 ? (uint32_t)blk : 0u) * 128u + 8u * (ln & 15);
                    uint32_t offk[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        offk[i] = (32 * (uint32_t)(wave & 3) + 8 * (ln >> 4) + (uint32_t)i) * (uint32_t)(2 * K) + 2 * lcol;
                    R[ld] = load_rows(x, K, I[ld], kt, offk);
                } else {
                    R[ld] = load_rows(x, K, I[ld], kt, off);
                }
                if (tt >= 3 && !wait_at_least(&drained[(tt - 3) % kSlots],
                                              kQConsumerWaves * ((tt - 3) / kSlots + 1), wc))
                    return;
                const uint32_t fl = flags_of(prev_sb, I[u], tt == 0 && run.lead);
                // slot tt % 4 of pmax is rewritten only in strip tt + 4, which starts after
                // the consumers drained strip tt + 1, so after every producer quantized
                // strip tt (and read its maxima before that)
                publish_col_max(R[u], tt % kSlots);
                signal(&colpub[wave]);
                const int wb = wave & ~3;
                if (!wait_at_least(&colpub[wb], tt + 1, wc) || !wait_at_least(&colpub[wb + 1], tt + 1, wc) ||
                    !wait_at_least(&colpub[wb + 2], tt + 1, wc) || !wait_at_least(&colpub[wb + 3], tt + 1, wc))
                    return;
                produce(I[u], R[u], tt % kSlots, fl);
                prev_sb = I[u].sb;
                signal(&produced[wave]);
                if constexpr (kRows)
                    produce_rows(I[u], R[u], fl);
                if (tt + 1 >= n)
                    return;
            }
        }
    }

    // ================= consumers =================
    consume_strips<kQConsumerWaves>(
        tile, info, drained, yT, ncols, n, wave - kQProducerWaves,
        [&](uint32_t t) { return wait_all_at_least<kQProducerWaves>(produced, t + 1, wc); },
        [&](uint32_t slot) {
            if (lane < 16 && 16 * lane < ncols)
                *reinterpret_cast<u32x4*>(yT_scales + K * (int64_t)uniform(info[slot].blk) +
                                          kTileCols * (int64_t)kt + 16 * lane) =
                    *reinterpret_cast<const u32x4*>(&sbytes[slot][16 * lane]);
        });
}

hipError_t launch_fp8q_cols(const uint16_t* x, uint8_t* yT, uint8_t* yT_scales, uint8_t* y, uint8_t* y_scales,
                            const int32_t* offs, int32_t G, int64_t M_cap, int64_t K, WaitCtl wc,
                            hipStream_t stream)
{
    if (M_cap == 0)
        return hipSuccess;
    const int64_t nkt = (K + kTileCols - 1) / kTileCols;
    // one workgroup per compute unit (the LDS ring takes most of a CU's LDS): parts per
    // column tile so that nkt * parts fills the GPU, never more parts than strips
    const int64_t cap_strips = (M_cap + kStripRows - 1) / kStripRows + G;
    int64_t parts = (int64_t)device_cus() / nkt;
    parts = parts < 1 ? 1 : parts;
    parts = parts > cap_strips ? cap_strips : parts;
    const int64_t grid = nkt * parts;
    if (grid > 0x7FFFFFFF)
        return hipErrorInvalidValue;
    const uint8_t* xb = reinterpret_cast<const uint8_t*>(x);
    int g = G;
    int64_t k = K;
    int p = (int)parts;
    void* args[] = {(void*)&xb, (void*)&yT, (void*)&yT_scales, (void*)&y, (void*)&y_scales, (void*)&offs,
                    (void*)&g, (void*)&k, (void*)&p, (void*)&wc};
    const void* kern = y ? (const void*)fp8q_cols_kernel<true> : (const void*)fp8q_cols_kernel<false>;
    return launch_kernel(kern, dim3((unsigned)grid), dim3(kQThreads), args, stream);
}

}  // namespace mxfp4
