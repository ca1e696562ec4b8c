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
// has M_g bytes, so the 128-token piece of a row starts at any byte.  The pieces go
// straight from memory into two 64 KB LDS buffers with buffer_load ... lds, whose
// 16-byte lanes take any byte alignment (checked on MI355X with an in-bounds probe: the
// bytes land as they are at a misaligned address), so no register staging or shifting
// is needed; LDS rows are 128 bytes with chunk c of row r at c ^ ((r >> 1) & 7), as in
// the forward GEMM, and the loop is software-pipelined the same way.  Bytes past token
// M_g in the last step belong to the next row: both operands' fragments are masked to
// zero there in registers, so the partial last block adds nothing.  Loads are buffer
// loads with the whole offset in the per-lane part, over the caller's capacity from the
// expert's first byte, so no access leaves the operand buffers.  The epilogue stages
// the BF16 tile in LDS and stores whole 512-byte row segments.
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
constexpr uint32_t kWGroupN = 2;                  // n tiles swept together (L2 reuse)

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

// What a wave needs in the step loop.
struct WgCtx {
    uint8_t* lds;                                 // two step buffers of kWStage bytes
    __amdgpu_buffer_rsrc_t rdy, rx;
    int wm, wn;
    uint32_t r, h;
};

// The fragments of one MFMA K-step (64 tokens) of a wave: two X^T tiles, four dY^T tiles.
struct WgFrag {
    wg_i32x8 x[2];
    wg_i32x8 d[4];
};

// A lane's fragment of one operand row: the row's 16-byte LDS chunks at c0 and c1.
__device__ __forceinline__ wg_i32x8 wg_frag(const uint8_t* rowp, uint32_t c0, uint32_t c1)
{
    const u32x4 v0 = *reinterpret_cast<const u32x4*>(rowp + c0);
    const u32x4 v1 = *reinterpret_cast<const u32x4*>(rowp + c1);
    return wg_i32x8{(int)v0.x, (int)v0.y, (int)v0.z, (int)v0.w, (int)v1.x, (int)v1.y, (int)v1.z, (int)v1.w};
}

// Where lane (r, h) reads K-step j of buffer b: tokens 64 j + 16 h .. + 15 and
// 64 j + 32 + 16 h .. + 15 of its rows (logical chunks 4 j + h and 4 j + 2 + h; LDS rows
// are 128 bytes with chunk c of row x at c ^ ((x >> 1) & 7)).
struct WgAddr {
    const uint8_t* td;
    const uint8_t* tx;
    uint32_t c0, c1;
};
__device__ __forceinline__ WgAddr wg_addr(const WgCtx& cx, uint32_t b, int j)
{
    const uint32_t sw8 = (cx.r >> 1) & 7;
    const uint8_t* const base = cx.lds + b * kWStage;
    return WgAddr{base + (128 * cx.wm + cx.r) * kWS, base + (kWT + 64 * cx.wn + cx.r) * kWS,
                  16 * ((4 * j + cx.h) ^ sw8), 16 * ((4 * j + 2 + cx.h) ^ sw8)};
}

__device__ __forceinline__ void wg_read(const WgCtx& cx, uint32_t b, int j, WgFrag& f)
{
    const WgAddr ad = wg_addr(cx, b, j);
#pragma unroll
    for (int q = 0; q < 2; ++q)
        f.x[q] = wg_frag(ad.tx + 32 * q * kWS, ad.c0, ad.c1);
#pragma unroll
    for (int q = 0; q < 4; ++q)
        f.d[q] = wg_frag(ad.td + 32 * q * kWS, ad.c0, ad.c1);
}

// Zero the bytes of tokens >= valid (counted from the step's first token) in the
// fragments of K-step j read by lane half h: dword e holds tokens
// 64 j + 16 h + 32 (e / 4) + 4 (e % 4) .. + 3.
__device__ __forceinline__ void wg_mask(WgFrag& f, int valid, int j, uint32_t h)
{
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int v = min(max(valid - (64 * j + 16 * (int)h + 32 * (e >> 2) + 4 * (e & 3)), 0), 4);
        const int m = v >= 4 ? -1 : (int)((1u << (8 * v)) - 1u);
#pragma unroll
        for (int q = 0; q < 2; ++q)
            f.x[q][e] &= m;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            f.d[q][e] &= m;
    }
}

// The eight MFMAs of one K-step on `cur`.  With kRead, K-step j of buffer b is read into
// `next` between them (the X^T tiles first, then one dY^T tile after each dY^T tile's
// MFMAs).  As in the forward GEMM, a wave raises its priority while it issues MFMAs.
template <bool kRead>
__device__ __forceinline__ void wg_step(const WgCtx& cx, const WgFrag& cur, const uint32_t (&sx)[2],
                                        const uint32_t (&sdy)[4], wg_f32x16 (&acc)[4][2], uint32_t b, int j,
                                        WgFrag& next)
{
    const WgAddr ad = wg_addr(cx, b, j);
    if (kRead) {
        next.x[0] = wg_frag(ad.tx, ad.c0, ad.c1);
        next.x[1] = wg_frag(ad.tx + 32 * kWS, ad.c0, ad.c1);
    }
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
            acc[mt][nt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(cur.x[nt], cur.d[mt], acc[mt][nt], 0, 0,
                                                                          0, (int)sx[nt], 0, (int)sdy[mt]);
        if (kRead)
            next.d[mt] = wg_frag(ad.td + 32 * mt * kWS, ad.c0, ad.c1);
    }
    __builtin_amdgcn_s_setprio(0);
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

    // loader role: instruction i of wave w fills LDS rows 32 w + 8 i .. + 7 of each
    // operand with the step's 128-byte pieces (LDS DMA takes any byte alignment, so a
    // piece lands as it is, whatever the row start); lane L takes row 32 w + 8 i + L / 8
    // and LDS chunk L % 8, that is chunk (L % 8) ^ ((row >> 1) & 7) of the piece
    uint32_t ld_dy[4], ld_x[4];                   // byte offsets of the lane's slices at step 0
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t lrow = (uint32_t)(32 * wave + 8 * i + (lane >> 3));
        const uint32_t gc = (uint32_t)(lane & 7) ^ ((lrow >> 1) & 7);
        ld_dy[i] = (uint32_t)(n0 + lrow) * Mg + 16 * gc;
        ld_x[i] = (uint32_t)(k0 + lrow) * Mg + 16 * gc;
    }
    // compute role: wave (wm, wn), lane (r, h)
    const int wm = wave & 1, wn = wave >> 1;
    const uint32_t r = (uint32_t)(lane & 31), h = (uint32_t)(lane >> 5);
    uint32_t soff_x[2], soff_dy[4];               // scale bytes of the lane's rows
#pragma unroll
    for (int q = 0; q < 4; ++q)
        soff_dy[q] = (uint32_t)(n0 + 128 * wm + 32 * q + r);
#pragma unroll
    for (int q = 0; q < 2; ++q)
        soff_x[q] = (uint32_t)(k0 + 64 * wn + 32 * q + r);
    const WgCtx cx{lds, rdy, rx, wm, wn, r, h};

    // The step's loads into buffer b.  The whole offset is in the per-lane part, so the
    // range of the resource bounds every access.
    auto issue = [&](uint32_t t, uint32_t b) {
        typedef __attribute__((address_space(3))) uint8_t lds_u8;
        lds_u8* const st = (lds_u8*)(lds + b * kWStage);
        const uint32_t step = t * kWS;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rdy, st + (32 * wave + 8 * i) * kWS, 16, ld_dy[i] + step, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, st + (kWT + 32 * wave + 8 * i) * kWS, 16, ld_x[i] + step, 0,
                                                     0, 0);
        }
    };
    // A 16-byte slice that runs past the end of a resource's range reads as zero as a
    // whole, its bytes inside the range too.  Only the last step's slices can reach past
    // an expert's data (every earlier step ends inside its row), and past the range only
    // in tiles that reach the end of the operand buffers (an expert that ends at the
    // capacity).  In those tiles a lane re-reads each fragment chunk of the last step
    // whose slice crossed the end as aligned dwords (each checked on its own; the range
    // is a multiple of 4) and shifts it into place, before the mask.
    const uint32_t rng_dy = (uint32_t)min((uint64_t)N * (uint64_t)(M_cap - m0), (uint64_t)0xFFFFFFFFu);
    const uint32_t rng_x = (uint32_t)min((uint64_t)K * (uint64_t)(M_cap - m0), (uint64_t)0xFFFFFFFFu);
    const bool tail_tile = (uint64_t)(n0 + kWT) * Mg + (uint64_t)T * kWS > rng_dy ||
                           (uint64_t)(k0 + kWT) * Mg + (uint64_t)T * kWS > rng_x;
    auto refetch = [&](__amdgpu_buffer_rsrc_t rs, uint32_t rng, uint32_t row, uint32_t lc, wg_i32x8& fr, int half) {
        const uint32_t o = row * Mg + (T - 1) * kWS + 16 * lc;
        if (o < rng && o + 16 > rng) {
            const uint32_t a0 = o & ~3u, sh = o & 3u;
            uint32_t wv[5];
#pragma unroll
            for (int j = 0; j < 5; ++j)
                wv[j] = __builtin_amdgcn_raw_buffer_load_b32(rs, (int)(a0 + 4 * j), 0, 0);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                fr[4 * half + j] = (int)__builtin_amdgcn_alignbyte(wv[j + 1], wv[j], sh);
        }
    };
    auto refetch_step = [&](WgFrag& fr, int j) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const uint32_t lc = 4 * j + 2 * half + h;                     // the chunk's tokens / 16
#pragma unroll
            for (int q = 0; q < 2; ++q)
                refetch(rx, rng_x, (uint32_t)(k0 + 64 * wn + 32 * q) + r, lc, fr.x[q], half);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                refetch(rdy, rng_dy, (uint32_t)(n0 + 128 * wm + 32 * q) + r, lc, fr.d[q], half);
        }
    };
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
        uint32_t sc_x[2], sc_dy[4];               // scale bytes of the step in flight
        load_scales(0, sc_x, sc_dy);
        issue(0, 0);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        issue(T > 1 ? 1 : 0, 1);                  // (with one step: in range, unused)
        WgFrag f;
        wg_read(cx, 0, 0, f);
        // Per step t in buffer u = t % 2, software-pipelined by MFMA K-step as in the
        // forward GEMM: the second K-step's fragments are read while the first K-step's
        // MFMAs issue; the barrier (every lane's loads of step t + 1 have landed, every
        // wave has read all of buffer u) sits before the second K-step's MFMAs, which
        // issue while step t + 1's first fragments are read.  Step t + 2 goes into buffer
        // u (on the second-to-last step that is the last step again: in range, unused).
        for (uint32_t t = 0; t + 1 < T; ++t) {
            const uint32_t u = t & 1;
            uint32_t nx_x[2], nx_dy[4];
            load_scales(t + 1, nx_x, nx_dy);
            WgFrag g;
            wg_step<true>(cx, f, sc_x, sc_dy, acc, u, 1, g);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            issue(min(t + 2, T - 1), u);
            wg_step<true>(cx, g, sc_x, sc_dy, acc, u ^ 1, 0, f);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                sc_dy[q] = nx_dy[q];
#pragma unroll
            for (int q = 0; q < 2; ++q)
                sc_x[q] = nx_x[q];
            __builtin_amdgcn_sched_barrier(0);
        }
        // the last step: its bytes past token M_g belong to the next row (or lie past
        // the capacity, where they read as zero); both operands are masked to zero there
        // in registers, so the partial block adds nothing
        {
            WgFrag g;
            wg_read(cx, (T - 1) & 1, 1, g);
            if (tail_tile) {
                refetch_step(f, 0);
                refetch_step(g, 1);
            }
            const int valid = (int)Mg - (int)(kWS * (T - 1));                  // 1 .. 128
            wg_mask(f, valid, 0, h);
            wg_mask(g, valid, 1, h);
            wg_step<false>(cx, f, sc_x, sc_dy, acc, 0, 0, g);
            wg_step<false>(cx, g, sc_x, sc_dy, acc, 0, 0, f);
        }
    }

    // epilogue through LDS, as in the forward GEMM: lane (r, h) of MFMA tile (mt, nt)
    // holds n = 128 wm + 32 mt + r and k = 64 wn + 32 nt + 8 q + 4 h + (0..3) in values
    // 4q .. 4q + 3.  The waves write their BF16 results into the LDS buffers (tile row x,
    // 512 bytes, at x * 512, the 16-byte chunk c of the row at chunk c ^ (x % 32)), then
    // every lane stores 16-byte pieces of whole rows.
    __builtin_amdgcn_s_waitcnt(0);                // the last (unused) loads have landed too
    __syncthreads();                              // every wave is done with the last step
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const wg_f32x16& v = acc[mt][nt];
                const wg_bf16x2 p0 = {(__bf16)v[4 * q + 0], (__bf16)v[4 * q + 1]};
                const wg_bf16x2 p1 = {(__bf16)v[4 * q + 2], (__bf16)v[4 * q + 3]};
                const uint32_t c = 8 * (uint32_t)wn + 4 * nt + q;
                *reinterpret_cast<u32x2*>(lds + (128 * wm + 32 * mt + r) * 512 + 16 * (c ^ r) + 8 * h) =
                    u32x2{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1)};
            }
    __syncthreads();
    {
        const uint32_t c = (uint32_t)tid & 31;
        uint16_t* const tile = dw + ((int64_t)g * N + n0) * K + k0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint32_t row = ((uint32_t)tid >> 5) + 16 * i;          // tile row 0 .. 255
            store_stream(reinterpret_cast<u32x4*>(tile + (int64_t)row * K + 8 * c),
                         *reinterpret_cast<const u32x4*>(lds + row * 512 + 16 * (c ^ (row & 31))));
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
