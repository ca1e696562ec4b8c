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
// Tile = one 128-row block of one expert x 128 columns, 256 threads:
//   stage A  thread (h = t>>7, m = t&127) loads 32 code bytes of row m (columns
//            64h..64h+63) and its two MX scales; a wave max + LDS gives the four
//            per-group block scales; the 64 codes are converted with the gap table
//            and written row-major (128 B per row) into a 16 KiB LDS tile;
//   stage B  thread (mb = l&7, kq = 8w + l>>3) reads a 16-row x 4-column patch as
//            16 dwords, transposes it in registers with v_perm_b32 (4x4 byte
//            transposes) and stores four 16-byte runs along m; lanes 8i..8i+7 cover
//            one contiguous 128-byte output row segment.
// LDS skew: 16-byte chunk c of logical row r lives at physical row P(r), chunk
// c ^ f(r), with f(r) = (r ^ (r>>4)) & 7 and P(r) = r ^ (((r>>3) ^ (r>>4)) & 1).
// Stage A's 16-byte writes (16 consecutive rows, one chunk) and stage B's dword
// reads (8 row groups x 8 columns) then hit distinct banks for both a 32-bank and a
// 64-bank LDS.
#include "common.h"

namespace mxfp4 {

__constant__ GapLut kColsGapLut = make_gap_lut();

constexpr int kTileRows = 128;
constexpr int kTileCols = 128;

__device__ __forceinline__ uint32_t skew_f(uint32_t r) { return (r ^ (r >> 4)) & 7u; }
__device__ __forceinline__ uint32_t skew_p(uint32_t r) { return r ^ (((r >> 3) ^ (r >> 4)) & 1u); }
// dword index of (logical row r, 16-byte chunk c, dword w in the chunk)
__device__ __forceinline__ uint32_t lds_dword(uint32_t r, uint32_t c, uint32_t w)
{
    return skew_p(r) * 32u + ((c ^ skew_f(r)) << 2) + w;
}

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

struct StageA {
    u32x4 ca, cb;     // 64 codes of one row: groups 2h and 2h+1 of the tile
    uint32_t s2;      // their two MX scale bytes
};

// Row m of block b of the expert starting at row0 (nothing is read past the expert).
__device__ __forceinline__ StageA load_rows(const uint8_t* __restrict__ codes,
                                            const uint8_t* __restrict__ scales, int64_t row,
                                            bool valid, int64_t K, int64_t k0, int h)
{
    StageA a{{0, 0, 0, 0}, {0, 0, 0, 0}, 0};
    if (valid) {
        const u32x4* cp = reinterpret_cast<const u32x4*>(codes + row * (K / 2) + k0 / 2 + 32 * h);
        a.ca = cp[0];
        a.cb = cp[1];
        a.s2 = *reinterpret_cast<const uint16_t*>(scales + row * (K / 32) + k0 / 32 + 2 * h);
    }
    return a;
}

template <int kStrip>
__global__ __launch_bounds__(kThreads) void fp8_cols_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    uint8_t* __restrict__ yT, uint8_t* __restrict__ yT_scales,
    const int32_t* __restrict__ offs, int G, int64_t K)
{
    __shared__ uint32_t tile[kTileRows * kTileCols / 4];
    __shared__ uint32_t lut[2 * (kMaxGap + 1)];
    __shared__ uint32_t wave_max[2][4];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const uint32_t nkt = (uint32_t)(K / kTileCols);
    const uint32_t L = xcd_remap(blockIdx.x, gridDim.x);
    const uint32_t Sidx = L / nkt;
    const uint32_t kt = L % nkt;

    int g;
    uint32_t Bg, Sg;
    if (!find_strip<kStrip>(offs, G, Sidx, g, Bg, Sg))
        return;                                   // uniform: every wave sees the same Sidx
    const int64_t row0 = offs[g];
    const int64_t Mg = (int64_t)offs[g + 1] - row0;
    const uint32_t nb_g = (uint32_t)((Mg + kTileRows - 1) / kTileRows);
    const uint32_t b0 = (Sidx - Sg) * kStrip;
    const uint32_t nblk = min((uint32_t)kStrip, nb_g - b0);
    const int64_t k0 = (int64_t)kt * kTileCols;

    if (tid < 2 * (kMaxGap + 1))
        lut[tid] = kColsGapLut.w[tid >> 1][tid & 1];

    const int h = tid >> 7;                       // column half: groups 2h, 2h+1
    const int m = tid & 127;
    const uint32_t mb = lane & 7;                 // stage B: rows 16mb..16mb+15
    const uint32_t kq = 8u * wave + (lane >> 3);  // stage B: columns 4kq..4kq+3
    uint8_t* const outT0 = yT + K * row0 + 16 * mb;

    StageA nxt = load_rows(codes, scales, row0 + (int64_t)kTileRows * b0 + m,
                           (int64_t)kTileRows * b0 + m < Mg, K, k0, h);
    for (uint32_t i = 0; i < nblk; ++i) {
        const uint32_t b = b0 + i;
        const int nr = (int)min<int64_t>(kTileRows, Mg - (int64_t)kTileRows * b);
        const StageA cur = nxt;
        if (i + 1 < nblk)                          // prefetch the next block of the strip
            nxt = load_rows(codes, scales, row0 + (int64_t)kTileRows * (b + 1) + m,
                            (int64_t)kTileRows * (b + 1) + m < Mg, K, k0, h);

        // ---- stage A: block scales, convert, row-major into LDS ----------------------
        uint32_t pk = (cur.s2 & 0xFFu) | ((cur.s2 & 0xFF00u) << 8);
#pragma unroll
        for (int dlt = 32; dlt >= 1; dlt >>= 1) {
            uint32_t o = __shfl_xor(pk, dlt, 64);
            pk = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, pk),
                                                                        __builtin_bit_cast(u16x2, o)));
        }
        if (lane == 0)
            wave_max[i & 1][wave] = pk;
        __syncthreads();                          // wave maxima visible; previous stage B done
        // waves 2h and 2h+1 hold rows 0..63 and 64..127 of column half h
        const u16x2 wm = __builtin_elementwise_max(__builtin_bit_cast(u16x2, wave_max[i & 1][2 * h]),
                                                   __builtin_bit_cast(u16x2, wave_max[i & 1][2 * h + 1]));
        {
            uint32_t da = min((uint32_t)wm.x - (cur.s2 & 0xFFu), (uint32_t)kMaxGap);
            uint32_t db = min((uint32_t)wm.y - (cur.s2 >> 8), (uint32_t)kMaxGap);
            uint32_t la0 = lut[2 * da], la1 = lut[2 * da + 1];
            uint32_t lb0 = lut[2 * db], lb1 = lut[2 * db + 1];
            u32x2 p0 = convert8(cur.ca.x, la0, la1), p1 = convert8(cur.ca.y, la0, la1);
            u32x2 p2 = convert8(cur.ca.z, la0, la1), p3 = convert8(cur.ca.w, la0, la1);
            u32x2 p4 = convert8(cur.cb.x, lb0, lb1), p5 = convert8(cur.cb.y, lb0, lb1);
            u32x2 p6 = convert8(cur.cb.z, lb0, lb1), p7 = convert8(cur.cb.w, lb0, lb1);
            const uint32_t r = (uint32_t)m, c0 = 4u * h;
            *reinterpret_cast<u32x4*>(&tile[lds_dword(r, c0 + 0, 0)]) = u32x4{p0.x, p0.y, p1.x, p1.y};
            *reinterpret_cast<u32x4*>(&tile[lds_dword(r, c0 + 1, 0)]) = u32x4{p2.x, p2.y, p3.x, p3.y};
            *reinterpret_cast<u32x4*>(&tile[lds_dword(r, c0 + 2, 0)]) = u32x4{p4.x, p4.y, p5.x, p5.y};
            *reinterpret_cast<u32x4*>(&tile[lds_dword(r, c0 + 3, 0)]) = u32x4{p6.x, p6.y, p7.x, p7.y};
        }
        __syncthreads();                          // tile complete

        // ---- block scales of this block: 128 bytes, S of group k / 32 -----------------
        if (tid < 8) {
            const int grp = tid >> 1;             // 16 bytes per thread, two threads per group
            const u16x2 hm = __builtin_elementwise_max(
                __builtin_bit_cast(u16x2, wave_max[i & 1][2 * (grp >> 1)]),
                __builtin_bit_cast(u16x2, wave_max[i & 1][2 * (grp >> 1) + 1]));
            const uint32_t w4 = ((grp & 1) ? (uint32_t)hm.y : (uint32_t)hm.x) * 0x01010101u;
            *reinterpret_cast<u32x4*>(yT_scales + K * (int64_t)(Bg + b) + k0 + 16 * tid) =
                u32x4{w4, w4, w4, w4};
        }

        // ---- stage B: 16 rows x 4 columns per thread, transposed, stored along m ------
        uint32_t R[16];
#pragma unroll
        for (int j = 0; j < 16; ++j)
            R[j] = tile[lds_dword(16u * mb + j, kq >> 2, kq & 3)];
        uint32_t T[4][4];                         // T[r][kk]: rows 4r..4r+3 of column 4kq+kk
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
            transpose4x4(R[4 * r4], R[4 * r4 + 1], R[4 * r4 + 2], R[4 * r4 + 3],
                         T[r4][0], T[r4][1], T[r4][2], T[r4][3]);
        const int nvalid = nr - 16 * (int)mb;     // rows of this thread's 16 that exist
        if (nvalid > 0) {
            uint8_t* outT = outT0 + (int64_t)kTileRows * b;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                uint8_t* dst = outT + (k0 + 4 * kq + kk) * Mg;
                u32x4 v = {T[0][kk], T[1][kk], T[2][kk], T[3][kk]};
                if (nvalid >= 16) {
                    *reinterpret_cast<u32x4_unaligned*>(dst) = v;
                } else {
                    uint32_t w[4] = {v.x, v.y, v.z, v.w};
                    for (int q = 0; q < nvalid; ++q)
                        dst[q] = (uint8_t)(w[q >> 2] >> (8 * (q & 3)));
                }
            }
        }
    }
}

#ifndef MXFP4_COLS_STRIP
#define MXFP4_COLS_STRIP 2
#endif
// consecutive 128-row blocks one workgroup converts for its column tile
constexpr int kColsStrip = MXFP4_COLS_STRIP;

int64_t cols_block_capacity(int64_t M_cap, int32_t G)
{
    return (M_cap + kTileRows - 1) / kTileRows + G;
}

// Strips of kColsStrip blocks over all experts: at most ceil(M_cap / (128 kStrip)) + G.
static int64_t cols_strip_capacity(int64_t M_cap, int32_t G)
{
    return (M_cap + kTileRows * kColsStrip - 1) / (kTileRows * kColsStrip) + G;
}

hipError_t launch_fp8_cols(const uint8_t* codes, const uint8_t* scales, uint8_t* yT,
                           uint8_t* yT_scales, const int32_t* offs, int32_t G, int64_t M_cap,
                           int64_t K, hipStream_t stream)
{
    int64_t nkt = K / kTileCols;
    int64_t grid = cols_strip_capacity(M_cap, G) * nkt;
    if (M_cap == 0)
        return hipSuccess;
    if (grid > 0x7FFFFFFF)
        return hipErrorInvalidValue;
    int g = G;
    int64_t k = K;
    void* args[] = {(void*)&codes, (void*)&scales, (void*)&yT, (void*)&yT_scales, (void*)&offs,
                    (void*)&g, (void*)&k};
    return hipLaunchKernel((const void*)fp8_cols_kernel<kColsStrip>, dim3((unsigned)grid),
                           dim3(kThreads), args, 0, stream);
}

}  // namespace mxfp4
