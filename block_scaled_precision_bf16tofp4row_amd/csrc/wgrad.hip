// wgrad.hip -- expert-grouped FP8 GEMM, weight gradient: the consumer of the transposed
// per-expert column layouts.
//
// Method: "Practical FP4 Training for Large-Scale MoE Models on Hopper GPUs", technical
// summary section 2: GEMMs stay in FP8 on the block-scaled pipeline (item 1), and the
// column conversion fuses the transpose into the Wgrad conversion over ragged experts
// with no padding (item 3).  For expert g with M_g tokens the weight gradient contracts
// over its tokens:
//     dW[g, n, k] = bf16( sum_{m < M_g} dY_g[m, n] X_g[m, k] )
// dY_g^T [N, M_g] and X_g^T [K, M_g] come in the column layout: expert g at byte
// width * offs[g], rows of M_g bytes; UE8M0 scales [nb_g, width] at byte width * B_g (B_g
// = 128-token blocks of the experts before g), one per (128-token block, row), the
// partial last block scaling only the tokens it has.  An expert with no tokens gets 0.
//
// gfx950 mapping: v_mfma_scale_f32_32x32x64_f8f6f4 as in the forward GEMM, contracting
// over tokens: a 128-token scale block is two MFMA K-steps with one scale byte per
// operand row.  X^T rows are the first operand and dY^T rows the second, so a lane's
// results are 4 consecutive k of one n (one 8-byte store into dW_g [N, K]).
//
// Work: a workgroup of 8 waves (two per SIMD, so one wave's matrix work covers the
// other's loads and LDS traffic) owns a 256 (n) x 256 (k) tile of one expert's dW and
// walks the expert's tokens in steps of 128; wave (wm, wn) computes n 128 wm .. + 127 x
// k 64 wn .. + 63 as 4 x 2 MFMA tiles (128 fp32 accumulators per lane).  A column row
// has M_g bytes, so the 128-token piece of a row starts at any byte: a thread loads the
// aligned 16 bytes at or below its 16-byte slice and the dword after them, and shifts
// them into place with v_alignbyte by the row start's offset mod 4 (fixed per row).
// Bytes past token M_g (the next row's) are masked to zero, so the partial last block
// adds nothing.  The realigned slices go through registers into two 64 KB LDS buffers
// (128-byte rows, chunk c of row r at c ^ ((r >> 1) & 7), as in the forward GEMM), the
// next step's loads in flight during the current step's matrix work.  Loads are buffer
// loads with the whole offset in the per-lane part, over the caller's capacity from the
// expert's first byte, so no access leaves the operand buffers.
#include "strips.h"

namespace mxfp4 {

namespace {

typedef int wg_i32x8 __attribute__((ext_vector_type(8)));
typedef float wg_f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 wg_bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWgThreads = 512;                   // 8 waves, two per SIMD
constexpr int kWT = 256;                          // n and k per workgroup tile
constexpr int kWS = 128;                          // tokens per step (one scale block)
constexpr int kWStage = 2 * kWT * kWS;            // bytes of one LDS buffer (64 KB)
constexpr uint32_t kWGroupN = 4;                  // n tiles swept together (L2 reuse)

// 128-token blocks of the experts before g, summed over one wave (uniform result).
__device__ __forceinline__ uint32_t wg_blocks_before(const int32_t* __restrict__ offs, int g)
{
    const int lane = threadIdx.x & 63;
    uint32_t s = 0;
    for (int e = lane; e < g; e += 64)
        s += (uint32_t)((offs[e + 1] - offs[e] + 127) >> 7);
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1)
        s += (uint32_t)__shfl_xor((int)s, d, 64);
    return uniform(s);
}

// The expert with the r-th most tokens (ties to the lower index), for G <= 64: lane e
// holds expert e's count and counts the experts ahead of it.
__device__ __forceinline__ int wg_expert_of_rank(const int32_t* __restrict__ offs, int G, uint32_t r)
{
    const int e = threadIdx.x & 63;
    const uint32_t me = e < G ? (uint32_t)(offs[e + 1] - offs[e]) : 0u;
    uint32_t rank = 0;
    for (int j = 0; j < G; ++j) {
        const uint32_t mj = (uint32_t)__shfl((int)me, j, 64);
        rank += (mj > me || (mj == me && j < e)) ? 1u : 0u;
    }
    const uint64_t hit = __ballot(e < G && rank == r);
    return (int)uniform((uint32_t)(__builtin_ffsll((long long)hit) - 1));
}

}  // namespace

__global__ __launch_bounds__(kWgThreads, 1) void fp8_wgrad_kernel(
    const uint8_t* __restrict__ dyT, const uint8_t* __restrict__ sdy, const uint8_t* __restrict__ xT,
    const uint8_t* __restrict__ sx, uint16_t* __restrict__ dw, const int32_t* __restrict__ offs, int G,
    int64_t M_cap, int64_t scale_blocks_cap, int64_t N, int64_t K)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kWStage];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // workgroup -> (expert, n tile, k tile).  An expert's work per tile is its token
    // count, so the experts go largest first (for G <= 64; in index order beyond), and
    // consecutive workgroups, which the dispatcher deals round-robin over the XCDs, are
    // one expert's tiles: every XCD works on every expert.  Within an expert the tiles
    // go in groups of kWGroupN n tiles across all k tiles.
    const uint32_t ntn = (uint32_t)(N / kWT), ktn = (uint32_t)(K / kWT);
    const uint32_t lin = blockIdx.x;
    const uint32_t per = ntn * ktn;
    const uint32_t rank = lin / per;
    const int g = G <= 64 ? wg_expert_of_rank(offs, G, rank) : (int)rank;
    const uint32_t rem = lin - rank * per;
    const uint32_t grp = rem / (kWGroupN * ktn);
    const uint32_t gn = min(kWGroupN, ntn - grp * kWGroupN);
    const uint32_t idx = rem - grp * kWGroupN * ktn;
    const int64_t n0 = (int64_t)kWT * (grp * kWGroupN + idx % gn);
    const int64_t k0 = (int64_t)kWT * (idx / gn);

    const int64_t m0 = uniform((uint32_t)offs[g]);
    const uint32_t Mg = uniform((uint32_t)(offs[g + 1] - offs[g]));
    const uint32_t Bg = wg_blocks_before(offs, g);
    const uint32_t T = (Mg + kWS - 1) / kWS;      // steps (scale blocks) of this expert

    // operand bytes from the expert's first byte to the end of the caller's capacity
    const __amdgpu_buffer_rsrc_t rdy = strip_rsrc(dyT + N * m0, (uint64_t)N * (uint64_t)(M_cap - m0));
    const __amdgpu_buffer_rsrc_t rx = strip_rsrc(xT + K * m0, (uint64_t)K * (uint64_t)(M_cap - m0));
    const __amdgpu_buffer_rsrc_t rsdy =
        strip_rsrc(sdy + N * (int64_t)Bg, (uint64_t)N * (uint64_t)(scale_blocks_cap - Bg));
    const __amdgpu_buffer_rsrc_t rsx =
        strip_rsrc(sx + K * (int64_t)Bg, (uint64_t)K * (uint64_t)(scale_blocks_cap - Bg));

    // loader role: thread t takes the 16-byte slice c = t & 7 of the step's piece of
    // local rows (t >> 3) + 64 i, i = 0..3, of both operands
    const uint32_t lrow = (uint32_t)(tid >> 3), lchunk = (uint32_t)(tid & 7);
    const uint32_t lds_w = lrow * kWS + 16 * (lchunk ^ ((lrow >> 1) & 7));   // + 64 i kWS
    uint32_t o_dy[4], o_x[4];                     // byte offset of the slice at step 0
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        o_dy[i] = (uint32_t)(n0 + lrow + 64 * i) * Mg + 16 * lchunk;
        o_x[i] = (uint32_t)(k0 + lrow + 64 * i) * Mg + 16 * lchunk;
    }
    // compute role: wave (wm, wn), lane (r, h)
    const int wm = wave & 1, wn = wave >> 1;
    const uint32_t r = (uint32_t)(lane & 31), h = (uint32_t)(lane >> 5);
    const uint32_t sw8 = (r >> 1) & 7;                                 // the swizzle of rows r + 32 x
    uint32_t soff_x[2], soff_dy[4];               // scale bytes of the lane's rows
#pragma unroll
    for (int q = 0; q < 4; ++q)
        soff_dy[q] = (uint32_t)(n0 + 128 * wm + 32 * q + r);
#pragma unroll
    for (int q = 0; q < 2; ++q)
        soff_x[q] = (uint32_t)(k0 + 64 * wn + 32 * q + r);

    u32x4 dq[4], xq[4];                           // staged slices (aligned 16 bytes)
    uint32_t de[4], xe[4];                        // and the dword after them
    auto load_tiles = [&](uint32_t t) {
        const uint32_t step = t * kWS;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t ad = (o_dy[i] + step) & ~3u, ax = (o_x[i] + step) & ~3u;
            dq[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rdy, (int)ad, 0, 0));
            de[i] = __builtin_amdgcn_raw_buffer_load_b32(rdy, (int)(ad + 16), 0, 0);
            xq[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, (int)ax, 0, 0));
            xe[i] = __builtin_amdgcn_raw_buffer_load_b32(rx, (int)(ax + 16), 0, 0);
        }
    };
    // realign the staged slices of step t, mask tokens >= M_g, write LDS buffer `buf`
    auto store_tiles = [&](uint32_t buf, uint32_t t) {
        const int valid = (int)Mg - (int)(t * kWS) - 16 * (int)lchunk;   // tokens in the slice
        uint32_t mask[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int v = min(max(valid - 4 * j, 0), 4);
            mask[j] = v >= 4 ? 0xFFFFFFFFu : ((1u << (8 * v)) - 1u);
        }
        uint8_t* const s_dy = lds + buf * kWStage;           // dY^T rows: bytes [0, 32 KB)
        uint8_t* const s_x = s_dy + kWT * kWS;                // X^T rows: bytes [32 KB, 64 KB)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t sd = o_dy[i] & 3, sx_ = o_x[i] & 3;          // step * 128 keeps the byte offset mod 4
            const u32x4 q = dq[i], p = xq[i];
            const u32x4 vd = {__builtin_amdgcn_alignbyte(q.y, q.x, sd) & mask[0],
                              __builtin_amdgcn_alignbyte(q.z, q.y, sd) & mask[1],
                              __builtin_amdgcn_alignbyte(q.w, q.z, sd) & mask[2],
                              __builtin_amdgcn_alignbyte(de[i], q.w, sd) & mask[3]};
            const u32x4 vx = {__builtin_amdgcn_alignbyte(p.y, p.x, sx_) & mask[0],
                              __builtin_amdgcn_alignbyte(p.z, p.y, sx_) & mask[1],
                              __builtin_amdgcn_alignbyte(p.w, p.z, sx_) & mask[2],
                              __builtin_amdgcn_alignbyte(xe[i], p.w, sx_) & mask[3]};
            *reinterpret_cast<u32x4*>(s_dy + lds_w + 64 * i * kWS) = vd;
            *reinterpret_cast<u32x4*>(s_x + lds_w + 64 * i * kWS) = vx;
        }
    };
    uint32_t sc_x[2], sc_dy[4];                   // current step's scale bytes
    uint32_t nx_x[2], nx_dy[4];
    auto load_scales = [&](uint32_t t, uint32_t (&dx)[2], uint32_t (&ddy)[4]) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            ddy[q] = __builtin_amdgcn_raw_buffer_load_b8(rsdy, (int)(soff_dy[q] + t * (uint32_t)N), 0, 0);
#pragma unroll
        for (int q = 0; q < 2; ++q)
            dx[q] = __builtin_amdgcn_raw_buffer_load_b8(rsx, (int)(soff_x[q] + t * (uint32_t)K), 0, 0);
    };

    wg_f32x16 acc[4][2];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
            acc[mt][nt] = wg_f32x16{};

    if (T > 0) {                                  // uniform: an empty expert writes zeros
        load_tiles(0);
        load_scales(0, sc_x, sc_dy);
        store_tiles(0, 0);
        __syncthreads();
        for (uint32_t t = 0; t < T; ++t) {
            // the next step (the last one again on the last step: in range, unused)
            const uint32_t tn = min(t + 1, T - 1);
            load_tiles(tn);
            load_scales(tn, nx_x, nx_dy);
            const uint8_t* const tdy = lds + (t & 1) * kWStage + (128 * wm) * kWS;
            const uint8_t* const tx = lds + (t & 1) * kWStage + kWT * kWS + (64 * wn) * kWS;
            __builtin_amdgcn_s_setprio(1);        // as in the forward GEMM: matrix work first
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                const uint32_t c0 = 16 * ((4 * kh + h) ^ sw8), c1 = 16 * ((4 * kh + 2 + h) ^ sw8);
                wg_i32x8 fx[2], fdy[4];
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const uint8_t* const rowp_x = tx + (32 * q + r) * kWS;
                    const u32x4 x0 = *reinterpret_cast<const u32x4*>(rowp_x + c0);
                    const u32x4 x1 = *reinterpret_cast<const u32x4*>(rowp_x + c1);
                    fx[q] = wg_i32x8{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                                     (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint8_t* const rowp_d = tdy + (32 * q + r) * kWS;
                    const u32x4 d0 = *reinterpret_cast<const u32x4*>(rowp_d + c0);
                    const u32x4 d1 = *reinterpret_cast<const u32x4*>(rowp_d + c1);
                    fdy[q] = wg_i32x8{(int)d0.x, (int)d0.y, (int)d0.z, (int)d0.w,
                                      (int)d1.x, (int)d1.y, (int)d1.z, (int)d1.w};
                }
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt)
                        acc[mt][nt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                            fx[nt], fdy[mt], acc[mt][nt], 0, 0, 0, (int)sc_x[nt], 0, (int)sc_dy[mt]);
            }
            __builtin_amdgcn_s_setprio(0);
            // the other buffer was last read in step t - 1, before the previous barrier
            store_tiles((t + 1) & 1, tn);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                sc_dy[q] = nx_dy[q];
#pragma unroll
            for (int q = 0; q < 2; ++q)
                sc_x[q] = nx_x[q];
            __syncthreads();
        }
    }

    // epilogue: lane (r, h) of MFMA tile (mt, nt) holds n = 128 wm + 32 mt + r and
    // k = 64 wn + 32 nt + 8 q + 4 h + (0..3) in values 4q .. 4q + 3
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        uint16_t* const yrow = dw + ((int64_t)g * N + n0 + 128 * wm + 32 * mt + r) * K + k0 + 64 * wn + 4 * h;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const wg_f32x16& v = acc[mt][nt];
                const wg_bf16x2 p0 = {(__bf16)v[4 * q + 0], (__bf16)v[4 * q + 1]};
                const wg_bf16x2 p1 = {(__bf16)v[4 * q + 2], (__bf16)v[4 * q + 3]};
                *reinterpret_cast<u32x2*>(yrow + 32 * nt + 8 * q) =
                    u32x2{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1)};
            }
    }
}

hipError_t launch_fp8_wgrad(const uint8_t* dyT, const uint8_t* sdy, const uint8_t* xT, const uint8_t* sx,
                            uint16_t* dw, const int32_t* offs, int32_t G, int64_t M_cap,
                            int64_t scale_blocks_cap, int64_t N, int64_t K, hipStream_t stream)
{
    const int64_t grid = (int64_t)G * (N / kWT) * (K / kWT);
    if (grid <= 0)
        return hipSuccess;
    if (grid > 0x7FFFFFFF)
        return hipErrorInvalidValue;
    int g = G;
    void* args[] = {(void*)&dyT, (void*)&sdy, (void*)&xT, (void*)&sx, (void*)&dw, (void*)&offs, (void*)&g,
                    (void*)&M_cap, (void*)&scale_blocks_cap, (void*)&N, (void*)&K};
    return launch_kernel((const void*)fp8_wgrad_kernel, dim3((unsigned)grid), dim3(kWgThreads), args, stream);
}

}  // namespace mxfp4
