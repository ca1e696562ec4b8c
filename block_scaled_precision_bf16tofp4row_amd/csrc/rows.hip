// rows.hip -- MXFP4 -> block-scaled FP8 E4M3 in row layout (FPROP operand), with no
// BF16 intermediate.
//
// Method: "Practical FP4 Training for Large-Scale MoE Models on Hopper GPUs",
// technical summary section 2, item 1: the four 32-element MXFP4 blocks of one
// 128-element FP8 block are aligned to their largest scale S, each sub-block's
// exponent shifted by the gap d = S - s, so values stay equal (exactly, while the
// shifted value is representable in E4M3; otherwise rounded to nearest even).  The
// FP8 block scale is the UE8M0 byte S.  This is the page's FP4RowToFP8Row (item 3).
//
// Layout: K is a multiple of 128, so FP8 blocks never cross a row and the matrix
// is a flat stream of 128-blocks: block b reads code bytes [64b, 64b+64) and the
// four scale bytes [4b, 4b+4) (one aligned dword), writes FP8 bytes [128b, 128b+128)
// and block-scale byte b.  A lane takes 8 code bytes (16 codes, half a sub-block)
// and writes 16 FP8 bytes, so a wave's code loads (512 B) and FP8 stores (1 KiB) are
// each one contiguous run.  The conversion is integer-only: the 8-entry byte table
// for the lane's gap (from a 14-entry LDS table) is indexed four codes at a time by
// one v_perm_b32.  The FP8 block-scale bytes of a workgroup (one per 128-block) are
// gathered in LDS and written as whole 16-byte pieces.
#include "common.h"

namespace mxfp4 {

template <int U>
__global__ __launch_bounds__(kThreads) void fp8_rows_kernel(
    const u32x2* __restrict__ codes, const uint32_t* __restrict__ scales4,
    u32x4* __restrict__ y, uint8_t* __restrict__ y_scales,
    const int32_t* __restrict__ offs, int G, int64_t K)
{
    __shared__ uint32_t lut[2 * (kMaxGap + 1)];
    // the workgroup's FP8 block-scale bytes, consecutive in y_scales
    constexpr int kScaleBytes = kThreads * U / 8;
    __shared__ __attribute__((aligned(16))) uint8_t sbuf[kScaleBytes];
    const int tid = threadIdx.x;
    const int64_t m_tot = offs[G];
    const int64_t nunits = m_tot * (K / 16);           // units of 16 codes (8 bytes)
    const int64_t base = (int64_t)blockIdx.x * (kThreads * U);
    // the loads go out before the gap table is staged and the barrier, so a workgroup's
    // first memory requests do not wait for its set-up
    u32x2 c[U];
    uint32_t sc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        int64_t idx = base + u * kThreads + tid;
        bool ok = idx < nunits;
        c[u] = ok ? load_stream(codes + idx) : u32x2{0, 0};
        sc[u] = ok ? scales4[idx >> 3] : 0u;
    }
    if (tid < 2 * (kMaxGap + 1))
        lut[tid] = gap_lut_word(tid);
    __syncthreads();
    if (base >= nunits)
        return;                                        // uniform over the workgroup
#pragma unroll
    for (int u = 0; u < U; ++u) {
        int64_t idx = base + u * kThreads + tid;
        if (idx >= nunits)
            continue;
        uint32_t s0 = sc[u] & 0xFF, s1 = (sc[u] >> 8) & 0xFF, s2 = (sc[u] >> 16) & 0xFF, s3 = sc[u] >> 24;
        uint32_t S = max(max(s0, s1), max(s2, s3));
        uint32_t j = ((uint32_t)idx >> 1) & 3;          // sub-block of this lane's 16 codes
        uint32_t s = (sc[u] >> (8 * j)) & 0xFF;
        uint32_t d = min(S - s, (uint32_t)kMaxGap);
        uint32_t lo = lut[2 * d], hi = lut[2 * d + 1];
        u32x2 a = convert8(c[u].x, lo, hi), bb = convert8(c[u].y, lo, hi);
        u32x4 o = {a.x, a.y, bb.x, bb.y};
        store_stream(y + idx, o);
        if ((idx & 7) == 0)
            sbuf[(u * kThreads + tid) >> 3] = (uint8_t)S;
    }
    // The block-scale bytes go out as whole 16-byte pieces (single-byte stores from every
    // eighth lane, spread over workgroups, would each be a partial write to memory).  The
    // last workgroup may end inside a piece: its bytes past m_tot * K / 128 stay untouched.
    __syncthreads();
    if (tid < kScaleBytes / 16) {
        const int64_t nb = nunits >> 3;
        const int64_t p = (base >> 3) + 16 * tid;
        if (p + 16 <= nb)
            store_stream(reinterpret_cast<u32x4*>(y_scales + p), *reinterpret_cast<const u32x4*>(sbuf + 16 * tid));
        else
            for (int q = 0; q < 16 && p + q < nb; ++q)
                y_scales[p + q] = sbuf[16 * tid + q];
    }
}

// 8-byte code units per thread (all loads issued before any conversion); two measured
// faster than one, three, four or eight on MI355X
constexpr int kRowsU = 2;

hipError_t launch_fp8_rows(const uint8_t* codes, const uint8_t* scales, uint8_t* y,
                           uint8_t* y_scales, const int32_t* offs, int32_t G, int64_t M_cap,
                           int64_t K, hipStream_t stream)
{
    int64_t nunits_cap = M_cap * (K / 16);
    int64_t per_block = (int64_t)kThreads * kRowsU;
    int64_t grid = (nunits_cap + per_block - 1) / per_block;
    if (grid == 0)
        return hipSuccess;
    if (grid > 0x7FFFFFFF)
        return hipErrorInvalidValue;
    const u32x2* cv = reinterpret_cast<const u32x2*>(codes);
    const uint32_t* sv = reinterpret_cast<const uint32_t*>(scales);
    u32x4* yv = reinterpret_cast<u32x4*>(y);
    int g = G;
    int64_t k = K;
    void* args[] = {(void*)&cv, (void*)&sv, (void*)&yv, (void*)&y_scales, (void*)&offs, (void*)&g, (void*)&k};
    return launch_kernel((const void*)fp8_rows_kernel<kRowsU>, dim3((unsigned)grid), dim3(kThreads), args,
                         stream);
}

}  // namespace mxfp4
