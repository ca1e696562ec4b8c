// cols.hip -- MXFP4 -> block-scaled FP8 E4M3 in transposed column layout (Wgrad
// operand), per expert over ragged token segments, transpose fused into the
// conversion.
//
// Method: "Practical FP4 Training for Large-Scale MoE Models on Hopper GPUs",
// technical summary section 2, item 3: the Wgrad kernel (FP4RowToFP8Col) fuses the
// transpose with the conversion to keep global traffic minimal, stages the
// transpose through a padded / skewed shared-memory layout against bank conflicts,
// and handles the ragged per-expert token counts without padding; the scale
// alignment is the one of item 1 applied along the token dimension: for each
// 128-row block of an expert and each 32-column group, the FP8 scale S is the max
// of the (up to 128) MX scales of the rows that exist, and each element is shifted
// by S - s of its own row.
//
// Output layout: expert g's transpose [K, M_g] starts at byte K*offs[g]; element
// (k, m') at k*M_g + m'.  Its block scales [nb_g, K] start at byte K*B_g, B_g the
// number of 128-row blocks of experts 0..g-1 (nb_h = ceil(M_h / 128)).
//
// Tile = 128 columns (four MX groups) x a strip of up to 256 rows (two FP8 blocks) of
// one expert, 256 threads:
//   stage A  thread (kc = lane & 3, rq) loads the 16 code bytes of group kc for rows
//            4rq..4rq+3 and their MX scale bytes; four consecutive lanes cover one row's
//            64 contiguous code bytes and 4 contiguous scale bytes.  The FP8 scale of
//            each (128-row block, group) is a DPP / cross-lane max inside the wave and
//            an LDS exchange between the block's two waves.  Each row is converted with
//            the gap table of its own scale, then 4x4 byte transposes (v_perm_b32) turn
//            4 rows x 32 columns into 32 dwords (4 rows of one column each), written
//            into an LDS tile that is k-major: one LDS row per output column k, holding
//            that column's 256 strip bytes in output order;
//   stage B  16 lanes per output row: lane c stores the 16-byte aligned chunk c of the
//            strip's output range [A, A + nrows).  The range's misalignment delta =
//            A & 15 becomes an unaligned 16-byte LDS read (gfx950 reads LDS at any
//            byte address), so every global store is an aligned 16-byte store and 16
//            lanes cover one contiguous 256-byte run.  Only the first and last chunk
//            of a strip can be partial; they are written one byte per lane.
// LDS skew: the tile row of column k starts at byte 288k + 64 (k >> 5); 32 rows of 288
// bytes span a whole number of bank cycles, so the 64-byte shift per MX group puts the
// stage-A dword writes of the four groups (16 rows each per wave) in 64 distinct
// banks.  This plays the role of the page's padded, skewed shared-memory layout.
#include "common.h"

namespace mxfp4 {

__constant__ GapLut kColsGapLut = make_gap_lut();

constexpr int kTileRows = 128;
// 4x4 byte transpose: a[i] holds bytes (row i, col 0..3); o[j] gets bytes (row 0..3, col j).
__device__ __forceinline__ void transpose4x4(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3,
                                             uint32_t& o0, uint32_t& o1, uint32_t& o2, uint32_t& o3)
{
    uint32_t t0 = perm(a1, a0, 0x05010400u);   // a0.0 a1.0 a0.1 a1.1
    uint32_t t1 = perm(a1, a0, 0x07030602u);   // a0.2 a1.2 a0.3 a1.3
    uint32_t u0 = perm(a3, a2, 0x05010400u);   // a2.0 a3.0 a2.1 a3.1
    uint32_t u1 = perm(a3, a2, 0x07030602u);   // a2.2 a3.2 a2.3 a3.3
    o0 = perm(u0, t0, 0x05040100u);
    o1 = perm(u0, t0, 0x07060302u);
    o2 = perm(u1, t1, 0x05040100u);
    o3 = perm(u1, t1, 0x07060302u);
}

// Which expert owns global strip index Sidx (each expert's row blocks are cut into
// strips of kStrip consecutive blocks)?  Every wave computes this on its own (no
// barrier): lanes take 64 experts at a time and scan both their block counts and
// their strip counts, then ballot.  Returns false when Sidx is past the last strip.
template <int kStrip>
__device__ __forceinline__ bool find_strip(const int32_t* __restrict__ offs, int G, uint32_t Sidx,
                                           int& g_out, uint32_t& Bg_out, uint32_t& Sg_out)
{
    const int lane = threadIdx.x & 63;
    uint32_t run_b = 0, run_s = 0;
    for (int g0 = 0; g0 < G; g0 += 64) {
        int h = g0 + lane;
        uint32_t nb = 0;
        if (h < G)
            nb = (uint32_t)(offs[h + 1] - offs[h] + 127) >> 7;
        uint32_t ns = (nb + kStrip - 1) / kStrip;
        uint32_t ib = nb, is = ns;
#pragma unroll
        for (int dlt = 1; dlt < 64; dlt <<= 1) {
            uint32_t ob = __shfl_up(ib, dlt, 64);
            uint32_t os = __shfl_up(is, dlt, 64);
            if (lane >= dlt) {
                ib += ob;
                is += os;
            }
        }
        uint32_t lo_s = run_s + is - ns;
        bool mine = h < G && ns > 0 && Sidx >= lo_s && Sidx < run_s + is;
        uint64_t mask = __ballot(mine);
        if (mask) {
            int src = __builtin_ctzll(mask);
            g_out = g0 + src;
            Bg_out = __shfl(run_b + ib - nb, src, 64);
            Sg_out = __shfl(lo_s, src, 64);
            return true;
        }
        run_b += __shfl(ib, 63, 64);
        run_s += __shfl(is, 63, 64);
    }
    return false;
}

// ---- tile geometry -------------------------------------------------------------------
constexpr int kTileCols = 128;                        // four MX groups
constexpr int kStripRows = 256;                       // two FP8 row blocks
constexpr int kStripBlocks = kStripRows / kTileRows;
constexpr int kLdsRowBytes = 16 + kStripRows + 16;    // front pad, data, back pad
constexpr int kLdsBytes = kTileCols * kLdsRowBytes + 64 * 3;
static_assert(kStripRows == 4 * 64, "stage A maps 64 quads of rows over the 4 waves");
static_assert((32 * (kLdsRowBytes / 4)) % 64 == 0, "32 tile rows must span a multiple of 64 banks");

__device__ __forceinline__ uint32_t lds_row(uint32_t k) { return kLdsRowBytes * k + 64 * (k >> 5); }

__device__ __forceinline__ uint32_t u16max2(uint32_t a, uint32_t b)
{
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                  __builtin_bit_cast(u16x2, b)));
}

__global__ __launch_bounds__(kThreads) void fp8_cols_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    uint8_t* __restrict__ yT, uint8_t* __restrict__ yT_scales,
    const int32_t* __restrict__ offs, int G, int64_t K)
{
    __shared__ __attribute__((aligned(16))) uint8_t tile[kLdsBytes];
    __shared__ uint32_t wave_max[4];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
    const uint32_t nkt = (uint32_t)(K / kTileCols);
    const uint32_t L = xcd_remap(blockIdx.x, gridDim.x);
    const uint32_t Sidx = L / nkt;
    const uint32_t kt = L % nkt;

    int g;
    uint32_t Bg, Sg;
    if (!find_strip<kStripBlocks>(offs, G, Sidx, g, Bg, Sg))
        return;                                      // uniform: every wave sees the same Sidx
    const int64_t row0 = offs[g];
    const int64_t Mg = (int64_t)offs[g + 1] - row0;
    const int64_t r_lo = (int64_t)(Sidx - Sg) * kStripRows;   // strip start, relative to row0
    const int nrows = (int)min<int64_t>(kStripRows, Mg - r_lo);

    // ---- stage A -----------------------------------------------------------------------
    const int kc = lane & 3;                         // MX group inside the tile
    const int rq = (lane >> 2) + 16 * wave;          // rows 4rq..4rq+3 of the strip
    const int64_t rbase = row0 + r_lo + 4 * rq;
    u32x4 c4[4];
    uint32_t s[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const bool ok = 4 * rq + i < nrows;
        const int64_t row = rbase + i;
        c4[i] = ok ? *reinterpret_cast<const u32x4*>(codes + row * (K / 2) + 64 * (int64_t)kt + 16 * kc)
                   : u32x4{0, 0, 0, 0};
        s[i] = ok ? (uint32_t)scales[row * (K / 32) + 4 * (int64_t)kt + kc] : 0u;
    }
    // max over the wave's 64 rows for each group: lanes kc, kc+4, ... (16 of them)
    uint32_t m = max(max(s[0], s[1]), max(s[2], s[3]));
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp((int)m, (int)m, 0x124, 0xF, 0xF, false));  // row_ror:4
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp((int)m, (int)m, 0x128, 0xF, 0xF, false));  // row_ror:8
    m = max(m, (uint32_t)__shfl_xor((int)m, 16, 64));
    m = max(m, (uint32_t)__shfl_xor((int)m, 32, 64));
    // lanes 0..3 now hold groups 0..3; pack them as four bytes for the partner wave
    const uint32_t packed = __builtin_amdgcn_readlane(m, 0) | (__builtin_amdgcn_readlane(m, 1) << 8) |
                            (__builtin_amdgcn_readlane(m, 2) << 16) | (__builtin_amdgcn_readlane(m, 3) << 24);
    if (lane == 0)
        wave_max[wave] = packed;
    __syncthreads();
    // block 0 = waves 0, 1; block 1 = waves 2, 3
    const uint32_t bmax = __builtin_amdgcn_readfirstlane(
        __builtin_bit_cast(uint32_t, __builtin_elementwise_max(
            __builtin_bit_cast(u8x4, wave_max[wave & 2]), __builtin_bit_cast(u8x4, wave_max[(wave & 2) + 1]))));
    const uint32_t S = (bmax >> (8 * kc)) & 0xFF;
    if (tid < 16) {                                  // block scales: 2 blocks x 128 columns
        const int blk = tid >> 3, piece = tid & 7;
        if (kTileRows * blk < nrows) {
            const uint32_t both = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(
                __builtin_bit_cast(u8x4, wave_max[2 * blk]), __builtin_bit_cast(u8x4, wave_max[2 * blk + 1])));
            const uint32_t w4 = ((both >> (8 * (piece >> 1))) & 0xFF) * 0x01010101u;
            *reinterpret_cast<u32x4*>(yT_scales + K * (int64_t)(Bg + r_lo / kTileRows + blk) +
                                      kTileCols * (int64_t)kt + 16 * piece) = u32x4{w4, w4, w4, w4};
        }
    }
    uint32_t F[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t d = min(S - s[i], (uint32_t)kMaxGap);
        const uint32_t lo = kColsGapLut.w[d][0], hi = kColsGapLut.w[d][1];
        u32x2 p0 = convert8(c4[i].x, lo, hi), p1 = convert8(c4[i].y, lo, hi);
        u32x2 p2 = convert8(c4[i].z, lo, hi), p3 = convert8(c4[i].w, lo, hi);
        F[i][0] = p0.x; F[i][1] = p0.y; F[i][2] = p1.x; F[i][3] = p1.y;
        F[i][4] = p2.x; F[i][5] = p2.y; F[i][6] = p3.x; F[i][7] = p3.y;
    }
    // column 32kc + 4q + kk: dword of rows 4rq..4rq+3 at strip byte 4rq of its LDS row
    const uint32_t wbase = lds_row(32 * kc) + 16 + 4 * rq;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        uint32_t o[4];
        transpose4x4(F[0][q], F[1][q], F[2][q], F[3][q], o[0], o[1], o[2], o[3]);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            *reinterpret_cast<uint32_t*>(tile + wbase + kLdsRowBytes * (4 * q + kk)) = o[kk];
    }
    __syncthreads();

    // ---- stage B: 16 lanes per output row, 4 rows per step, 32 rows per wave ---------
    // Output row k of expert g starts at byte K*offs[g] + k*M_g; the strip's bytes are
    // [A, A + nrows) with A = that + r_lo.  Chunk c is memory [A - delta + 16c, +16)
    // with delta = A & 15, i.e. strip bytes [16c - delta, 16c - delta + 16).
    const int c = lane & 15;
#pragma unroll 2
    for (int it = 0; it < 8; ++it) {
        const uint32_t kl = 32 * wave + 4 * it + (lane >> 4);
        const int64_t A = K * row0 + (kTileCols * (int64_t)kt + kl) * Mg + r_lo;
        const int delta = (int)(A & 15);
        uint8_t* const C0 = yT + (A - delta);
        const int c_first = delta > 0 ? 1 : 0;         // first full chunk
        const int c_end = (delta + nrows) >> 4;         // one past the last full chunk
        const uint8_t* rowp = tile + lds_row(kl) + 16 - delta;   // rowp[16c + p] = chunk byte p
        if (c >= c_first && c < c_end)
            *reinterpret_cast<u32x4*>(C0 + 16 * (int64_t)c) =
                *reinterpret_cast<const u32x4_unaligned*>(rowp + 16 * c);
        // partial chunks (head: chunk 0 when delta > 0; tail: chunk c_end when the range
        // does not end on a chunk boundary; one chunk when the range is that short):
        // lane c writes byte c of each, if it belongs to the strip
        const bool head = delta > 0;
        const bool tail = ((delta + nrows) & 15) != 0 && !(head && c_end == 0);
        if (head && c >= delta && c - delta < nrows)
            C0[c] = rowp[c];
        const int ti = 16 * c_end + c;                 // byte of the tail chunk
        if (tail && ti >= delta && ti - delta < nrows)
            C0[ti] = rowp[ti];
    }
}

int64_t cols_block_capacity(int64_t M_cap, int32_t G)
{
    return (M_cap + kTileRows - 1) / kTileRows + G;
}

// Strips of kStripRows rows over all experts: at most ceil(M_cap / kStripRows) + G.
static int64_t cols_strip_capacity(int64_t M_cap, int32_t G)
{
    return (M_cap + kStripRows - 1) / kStripRows + G;
}

hipError_t launch_fp8_cols(const uint8_t* codes, const uint8_t* scales, uint8_t* yT,
                           uint8_t* yT_scales, const int32_t* offs, int32_t G, int64_t M_cap,
                           int64_t K, hipStream_t stream)
{
    int64_t grid = cols_strip_capacity(M_cap, G) * (K / kTileCols);
    if (M_cap == 0)
        return hipSuccess;
    if (grid > 0x7FFFFFFF)
        return hipErrorInvalidValue;
    int g = G;
    int64_t k = K;
    void* args[] = {(void*)&codes, (void*)&scales, (void*)&yT, (void*)&yT_scales, (void*)&offs,
                    (void*)&g, (void*)&k};
    return hipLaunchKernel((const void*)fp8_cols_kernel, dim3((unsigned)grid), dim3(kThreads), args,
                           0, stream);
}

}  // namespace mxfp4
