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
// Producers (waves 0-7): wave w quantizes rows 16w..16w+15 of every strip.  Lane
// (rq = lane >> 4, cc = lane & 15) holds rows 16w + 4rq .. + 3 of tile columns
// 8cc..8cc+7 and 128+8cc..128+8cc+7: sixteen lanes read one row's two 256-byte halves,
// so every load instruction reads whole 128-byte lines.  Loads run kQPrefetch strips
// ahead.  The column amax is reduced over the lane's four rows (packed 16-bit max on
// the magnitude bits), over the four row quads (lane shuffles), and over the eight
// waves (each publishes its partial maxima in LDS, every lane then takes the max of
// the eight for its sixteen columns).
// The element convert, v_cvt_scalef32_pk_fp8_bf16, takes one scale for a pair of
// BF16, and neighbouring columns have different scales, so a pair is two rows of one
// column (one v_perm_b32): the two converts of a column's four rows then give the
// column's ring dword directly, rows in order, with no byte transpose.  As in the row
// quantizer, magnitudes are clamped to 448 * 2^(S-127) before the convert (it returns
// NaN for quotients of 464 or more instead of saturating).
// Consumers (waves 8-15): strips.h.
#include "strips.h"

namespace mxfp4 {

typedef __bf16 qbf16x2 __attribute__((ext_vector_type(2)));

#ifndef MXFP4_FP8QC_CONSUMERS
#define MXFP4_FP8QC_CONSUMERS 8
#endif
#ifndef MXFP4_FP8QC_PREFETCH
#define MXFP4_FP8QC_PREFETCH 1
#endif
constexpr int kQProducerWaves = 8;                          // 16 rows each
constexpr int kQConsumerWaves = MXFP4_FP8QC_CONSUMERS;
constexpr int kQPrefetch = MXFP4_FP8QC_PREFETCH;            // strips of loads in flight
constexpr int kQThreads = 64 * (kQProducerWaves + kQConsumerWaves);
constexpr int kPmaxSlots = 2;                               // partial maxima: strips t and t + 1
static_assert(kStripRows == 16 * kQProducerWaves, "a producer wave quantizes 16 rows");
static_assert(kTileCols == 256, "a producer lane holds columns 8cc.. and 128 + 8cc..");
static_assert((kRing & (kRing - 1)) == 0, "the ring position wraps with a mask");

namespace {

// A lane's four rows of a strip, two 16-byte chunks (8 BF16) per row: v[i][h] holds
// tile columns 128h + 8cc .. + 7 of row 4rq + i of the wave's rows.
struct QRows {
    u32x4 v[4][2];
};

// Loads are unconditional (rows past the strip repeat its last row, which leaves the
// column amax unchanged; their converted bytes are never written out), so every strip
// issues the same straight-line sequence of loads.  Row offsets within a strip fit in
// 32 bits (128 rows x 2K bytes with K <= 2^24).
__device__ __forceinline__ QRows load_rows(const uint8_t* __restrict__ x, int64_t K, const StripInfo& st,
                                           int row_q, uint32_t cbyte0, uint32_t cbyte1, uint32_t kt)
{
    QRows in;
    const uint8_t* const xb = x + (st.row0 + st.r_lo) * (2 * K) + 512 * (int64_t)kt;
    const uint32_t rb = (uint32_t)(2 * K);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t r = (uint32_t)min(row_q + i, st.nrows - 1);
        in.v[i][0] = *reinterpret_cast<const u32x4*>(xb + (r * rb + cbyte0));
        in.v[i][1] = *reinterpret_cast<const u32x4*>(xb + (r * rb + cbyte1));
    }
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

__global__ __launch_bounds__(kQThreads, 1) void fp8q_cols_kernel(
    const uint8_t* __restrict__ x, uint8_t* __restrict__ yT, uint8_t* __restrict__ yT_scales,
    const int32_t* __restrict__ offs, int G, int64_t K, int parts)
{
    __shared__ __attribute__((aligned(16))) uint8_t tile[kTileBytes];
    __shared__ __attribute__((aligned(16))) SlotInfo info[kSlots];
    // per ring slot: the block scale byte of each tile column
    __shared__ __attribute__((aligned(16))) uint8_t sbytes[kSlots][kTileCols];
    // per strip parity, per producer wave: the largest BF16 magnitude field of each
    // tile column over the wave's 16 rows
    __shared__ __attribute__((aligned(16))) uint16_t pmax[kPmaxSlots][kQProducerWaves][kTileCols];
    __shared__ uint32_t produced, published, drained[kSlots];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t nkt = (uint32_t)((K + kTileCols - 1) / kTileCols);
    const uint32_t lambda = xcd_remap(blockIdx.x, gridDim.x);
    const uint32_t kt = lambda % nkt;
    const uint32_t part = lambda / nkt;
    const int ncols = (int)min<int64_t>(kTileCols, K - (int64_t)kTileCols * kt);

    const ExpertTable t0 = expert_chunk(offs, G, 0, 0);
    uint32_t n_strips = t0.total;
    for (int g0 = 64; g0 < G; g0 += 64)
        n_strips = uniform(n_strips + expert_chunk(offs, G, g0, n_strips).total);
    const uint32_t s0 = (uint32_t)(((uint64_t)n_strips * part) / (uint32_t)parts);
    const uint32_t s1 = (uint32_t)(((uint64_t)n_strips * (part + 1)) / (uint32_t)parts);
    if (s0 >= s1)
        return;                                   // uniform over the workgroup
    // a range that starts inside an expert also quantizes the strip before it (a
    // lead-in strip that writes nothing), so its first output line is written whole
    const StripInfo first = locate(offs, G, t0, s0);
    const uint32_t lead = first.s > first.sb ? 1u : 0u;
    const uint32_t n = s1 - s0 + lead;

    if (tid == 0) {
        produced = 0;
        published = 0;
        for (int k = 0; k < kSlots; ++k)
            drained[k] = 0;
    }
    __syncthreads();                              // the only barrier: counters set

    if (wave < kQProducerWaves) {
        // ================= producers =================
        const int cc = lane & 15;
        const int rq = lane >> 4;
        const int row_q = 16 * wave + 4 * rq;     // first of the lane's four rows
        // the narrow last tile (128 columns) has no second half: those lanes repeat the
        // first half (their columns are never written out)
        const uint32_t cbyte0 = 16 * (uint32_t)cc;
        const uint32_t cbyte1 = ncols > 128 ? 256 + cbyte0 : cbyte0;
        // tile column 128h + 8cc + j sits at LDS byte lds_col(128h + 8cc) + 544 j
        const uint32_t wbase0 = lds_col(8 * cc) + row_q;
        const uint32_t wbase1 = lds_col(128 + 8 * cc) + row_q;

        // this wave's partial maxima of strip `st` (its 16 rows) into pmax[ps]
        auto publish_max = [&](const QRows& in, uint32_t ps) {
            uint32_t m[2][4];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const u32x4 a = in.v[0][h], b = in.v[1][h], c = in.v[2][h], d = in.v[3][h];
                m[h][0] = pk_max_u16(pk_max_u16(a.x & 0x7FFF7FFFu, b.x & 0x7FFF7FFFu),
                                     pk_max_u16(c.x & 0x7FFF7FFFu, d.x & 0x7FFF7FFFu));
                m[h][1] = pk_max_u16(pk_max_u16(a.y & 0x7FFF7FFFu, b.y & 0x7FFF7FFFu),
                                     pk_max_u16(c.y & 0x7FFF7FFFu, d.y & 0x7FFF7FFFu));
                m[h][2] = pk_max_u16(pk_max_u16(a.z & 0x7FFF7FFFu, b.z & 0x7FFF7FFFu),
                                     pk_max_u16(c.z & 0x7FFF7FFFu, d.z & 0x7FFF7FFFu));
                m[h][3] = pk_max_u16(pk_max_u16(a.w & 0x7FFF7FFFu, b.w & 0x7FFF7FFFu),
                                     pk_max_u16(c.w & 0x7FFF7FFFu, d.w & 0x7FFF7FFFu));
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    m[h][q] = pk_max_u16(m[h][q], (uint32_t)__shfl_xor((int)m[h][q], 16, 64));
                    m[h][q] = pk_max_u16(m[h][q], (uint32_t)__shfl_xor((int)m[h][q], 32, 64));
                }
            }
            if (rq == 0) {
                *reinterpret_cast<u32x4*>(&pmax[ps][wave][8 * cc]) = u32x4{m[0][0], m[0][1], m[0][2], m[0][3]};
                *reinterpret_cast<u32x4*>(&pmax[ps][wave][128 + 8 * cc]) =
                    u32x4{m[1][0], m[1][1], m[1][2], m[1][3]};
            }
        };

        auto produce = [&](const StripInfo& st, const QRows& in, uint32_t slot, uint32_t ps, uint32_t flags) {
            // column maxima over the strip: max of the eight waves' partial maxima
            uint32_t M[2][4];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                u32x4 acc = *reinterpret_cast<const u32x4*>(&pmax[ps][0][128 * h + 8 * cc]);
#pragma unroll
                for (int w = 1; w < kQProducerWaves; ++w) {
                    const u32x4 o = *reinterpret_cast<const u32x4*>(&pmax[ps][w][128 * h + 8 * cc]);
                    acc = u32x4{pk_max_u16(acc.x, o.x), pk_max_u16(acc.y, o.y), pk_max_u16(acc.z, o.z),
                                pk_max_u16(acc.w, o.w)};
                }
                M[h][0] = acc.x;
                M[h][1] = acc.y;
                M[h][2] = acc.z;
                M[h][3] = acc.w;
            }
            // scale bytes: biased exponent field of the column max minus 8, at least 0
            uint32_t Sb[2][2];            // [h][columns 0..3 / 4..7] as bytes
#pragma unroll
            for (int h = 0; h < 2; ++h) {
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    const u16x2 e0 = __builtin_bit_cast(u16x2, M[h][2 * p]) >> (unsigned short)7;
                    const u16x2 e1 = __builtin_bit_cast(u16x2, M[h][2 * p + 1]) >> (unsigned short)7;
                    const u16x2 eight = {8, 8};
                    const u16x2 s0v = __builtin_elementwise_sub_sat(e0, eight);
                    const u16x2 s1v = __builtin_elementwise_sub_sat(e1, eight);
                    Sb[h][p] = (uint32_t)s0v.x | ((uint32_t)s0v.y << 8) | ((uint32_t)s1v.x << 16) |
                               ((uint32_t)s1v.y << 24);
                }
            }
            if (wave == 0) {
                if (rq == 0) {
                    *reinterpret_cast<u32x2*>(&sbytes[slot][8 * cc]) = u32x2{Sb[0][0], Sb[0][1]};
                    *reinterpret_cast<u32x2*>(&sbytes[slot][128 + 8 * cc]) = u32x2{Sb[1][0], Sb[1][1]};
                }
                if (lane == 0) {
                    info[slot].A0 = K * st.row0 + st.r_lo + (int64_t)kTileCols * kt * st.mg;
                    info[slot].mg = (int32_t)st.mg;
                    info[slot].nrows = st.nrows;
                    info[slot].blk = st.s;
                    info[slot].flags = flags;
                }
            }
            // quantize column by column: rows (0, 1) and (2, 3) of the lane's four rows
            // form the two pairs of one convert each; the result dword is the column's
            // four ring bytes in row order
            const uint32_t sl = kStripRows * slot;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                uint8_t* const w = tile + (h ? wbase1 : wbase0) + sl;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const uint32_t S = (Sb[h][j >> 2] >> (8 * (j & 3))) & 0xFFu;
                    const uint32_t clamp = ((S + 8) << 7) | 0x60u;
                    const uint32_t clamp2 = clamp * 0x00010001u;
                    const float scale = __uint_as_float(S == 0 ? 0x00400000u : S << 23);
                    const int q = j >> 1;
                    const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
                    const uint32_t r01 = perm(in.v[1][h][q], in.v[0][h][q], sel);
                    const uint32_t r23 = perm(in.v[3][h][q], in.v[2][h][q], sel);
                    u16x2 acc = {0, 0};
                    acc = cvt_pair<false>(acc, r01, clamp2, scale);
                    acc = cvt_pair<true>(acc, r23, clamp2, scale);
                    const uint32_t T = __builtin_bit_cast(uint32_t, acc);
                    *reinterpret_cast<uint32_t*>(w + kColBytes * j) = T;
                    // ring bytes 0..31 (rows 0..31 of slot 0, waves 0 and 1) are repeated
                    // after the ring, so a 32-byte read window never wraps
                    if (slot == 0 && wave < 2)
                        *reinterpret_cast<uint32_t*>(w + kRing + kColBytes * j) = T;
                }
            }
        };
        auto flags_of = [](uint32_t prev_sb, const StripInfo& cur, bool lead_in) {
            return (prev_sb == cur.sb ? 1u : 0u) | (cur.s + 1 < cur.sb + cur.ns ? 2u : 0u) | (lead_in ? 4u : 0u);
        };

        // Step t waits until the consumers have drained strip t - 3 (whose slot carries
        // into strip t - 2, the last reader of slot t % 4) and until all producer waves
        // have published their partial maxima of strip t, quantizes strip t, signals it,
        // and publishes its own partial maxima of strip t + 1.  Register sets rotate over
        // kQPrefetch + 1 strips; the loop is unrolled by that much so each set keeps
        // fixed registers.
        constexpr int kSets = kQPrefetch + 1;
        uint32_t prev_sb = 0xFFFFFFFFu;
        StripInfo I[kSets];
        QRows R[kSets];
        I[0] = first;
        I[0].s -= lead;
        set_rows(I[0]);
#pragma unroll
        for (int u = 1; u < kQPrefetch; ++u)
            I[u] = (uint32_t)u < n ? next_strip(offs, G, I[u - 1]) : I[u - 1];
#pragma unroll
        for (int u = 0; u < kQPrefetch; ++u)
            R[u] = load_rows(x, K, I[u], row_q, cbyte0, cbyte1, kt);
        publish_max(R[0], 0);
        signal(&published);
        for (uint32_t t = 0;; t += kSets) {
#pragma unroll
            for (int u = 0; u < kSets; ++u) {
                const uint32_t tt = t + u;
                const int ld = (u + kQPrefetch) % kSets;          // set receiving strip tt + kQPrefetch
                const int pv = (u + kQPrefetch - 1) % kSets;      // set of strip tt + kQPrefetch - 1
                I[ld] = tt + kQPrefetch < n ? next_strip(offs, G, I[pv]) : I[pv];
                R[ld] = load_rows(x, K, I[ld], row_q, cbyte0, cbyte1, kt);
                const int nx = (u + 1) % kSets;                   // set of strip tt + 1
                if (tt >= 3 && !wait_at_least(&drained[(tt - 3) % kSlots],
                                              kQConsumerWaves * ((tt - 3) / kSlots + 1)))
                    return;
                if (!wait_at_least(&published, kQProducerWaves * (tt + 1)))
                    return;
                produce(I[u], R[u], tt % kSlots, tt % kPmaxSlots, flags_of(prev_sb, I[u], tt == 0 && lead != 0));
                prev_sb = I[u].sb;
                signal(&produced);
                if (tt + 1 >= n)
                    return;
                publish_max(R[nx], (tt + 1) % kPmaxSlots);
                signal(&published);
            }
        }
    }

    // ================= consumers =================
    consume_strips<kQProducerWaves, kQConsumerWaves>(
        tile, info, &produced, drained, yT, ncols, n, wave - kQProducerWaves, [&](uint32_t slot) {
            if (lane < 16 && 16 * lane < ncols)
                *reinterpret_cast<u32x4*>(yT_scales + K * (int64_t)uniform(info[slot].blk) +
                                          kTileCols * (int64_t)kt + 16 * lane) =
                    *reinterpret_cast<const u32x4*>(&sbytes[slot][16 * lane]);
        });
}

hipError_t launch_fp8q_cols(const uint16_t* x, uint8_t* yT, uint8_t* yT_scales, const int32_t* offs,
                            int32_t G, int64_t M_cap, int64_t K, hipStream_t stream)
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
    void* args[] = {(void*)&xb, (void*)&yT, (void*)&yT_scales, (void*)&offs, (void*)&g, (void*)&k, (void*)&p};
    return hipLaunchKernel((const void*)fp8q_cols_kernel, dim3((unsigned)grid), dim3(kQThreads), args, 0,
                           stream);
}

}  // namespace mxfp4
