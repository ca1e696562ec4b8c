// gemm.hip -- expert-grouped FP8 GEMM, forward (row layout): the FP8 compute step that
// consumes the converted activations.
//
// Method: "Practical FP4 Training for Large-Scale MoE Models on Hopper GPUs", technical
// summary section 2: GEMMs run in FP8 on the standard block-scaled pipeline (item 1:
// E4M3 with 128-element blocks; storage and communication are FP4, compute is FP8); the
// forward expert GEMM takes the row-layout FP8 activations produced by the direct
// FP4 -> FP8 conversion.  For the expert g that owns row m (offs[g] <= m < offs[g+1]):
//     y[m, n] = bf16( sum_k A[m,k] 2^(sA[m,k/128]-127) * W_g[n,k] 2^(sW_g[n,k/128]-127) )
// A [M, K] and W_g [N, K] are E4M3 with one UE8M0 scale per 1x128 block along K.
//
// gfx950 mapping: v_mfma_scale_f32_32x32x64_f8f6f4 multiplies a 32x64 by a 64x32 E4M3
// block and applies one E8M0 scale per 32 K-elements of each operand row in the
// hardware, so the 1x128 block scales cost nothing: a lane passes the scale of its
// row's current 128-block.  Operand layout (measured on MI355X with an in-bounds probe):
// lane l supplies row l % 32; bytes 0-15 of its 32 are K-block 0 (k < 32) and bytes
// 16-31 K-block 1; which k within a block a byte is does not matter as long as both
// operands agree, so lane (r, h = l / 32) takes k in [16h, 16h + 16) and
// [32 + 16h, 32 + 16h + 16); its scale byte applies to (row r, K-block h).  Result
// value i of lane l is row (i / 4) * 8 + (l / 32) * 4 + i % 4, column l % 32.  With the
// weights as the first operand and the tokens as the second, a lane's results are 4
// consecutive output features of one token (one 8-byte store).
//
// Work (K a multiple of 256 up to 7168, the fast path): a workgroup of 8 waves (two
// per SIMD, so one wave's matrix work hides the other's LDS reads) owns a 256-token x
// 256-feature tile of one expert and walks K in stages of 128 (one scale block);
// wave (wm, wn) computes tokens 128 wm .. + 127 x features 64 wn .. + 63 as 4 x 2
// MFMA tiles (128 fp32 accumulators per lane), two MFMA K-steps per stage.  Operand
// tiles go straight from memory to LDS (buffer_load ... lds: lane L's 16 bytes land at
// the instruction's LDS base + 16 L) into two 64 KB buffers, the next stage's loads
// running during the current stage's matrix work, with no registers held for them.
// Each wave loads 32 rows of each operand per stage, 8 rows x 128 bytes (whole cache
// lines) per instruction; LDS rows are 128 bytes with the 16-byte chunk c of row r
// stored at chunk c ^ ((r >> 1) & 7), so the fragment reads of 16 consecutive rows
// (one LDS cycle of a 16-byte read) hit distinct banks (a lane of the load picks the
// global chunk that belongs in its LDS slot).  The compiler does not see that the
// fragment reads depend on these loads, so a stage is awaited explicitly: before the
// barrier that opens stage t + 1 a lane waits for its own loads of it.  The loop is
// software-pipelined by MFMA K-step: that barrier sits between the second K-step's
// fragment reads of stage t and its MFMAs, so after it every wave has eight MFMAs
// queued on registers it already holds while it reads stage t + 1's first fragments
// (and the first K-step's MFMAs cover the second K-step's reads the same way).  Stages
// run in pairs (one per buffer) whose load issues are fixed at compile time, the last
// pair peeled, so that a pair is one basic block and the compiler keeps each stage's
// matrix work in its stage instead of sinking it towards the stores.  A wave raises its
// priority while it issues MFMAs (s_setprio), so the SIMD's other wave does its waiting
// meanwhile instead of both contending for the issue slots in lockstep.  The epilogue
// stages the BF16 tile in the free LDS buffers and stores whole 512-byte row segments.
// The tile's block scales (256 rows x K/128 bytes per operand) are staged in LDS once,
// laid out so that one 4-byte read gives a lane the scales of its four MFMA tiles; they
// take no registers across stages and no place in the memory-operation count.  Their
// loads (one dword per four blocks, all independent) go out together with stage 0's
// operand loads, so a workgroup's start waits for one memory round trip, not one per
// scale byte.  Operand
// and scale loads are buffer loads whose range is the tile's rows that exist: rows past
// the last partial tile of an expert read as zero (they add nothing), and the output
// stores go through a resource of the same rows, so those rows are never written.  The
// tile -> (expert, token tile) map is found on the device from the offsets.
// For other K (above 7168 the scales do not fit in LDS beside the buffers) a general
// kernel of 4 waves keeps the same workgroup tiles (128 x 128 per wave) with two 128-K
// register-staged LDS buffers and per-step scale loads.
#include "strips.h"

namespace mxfp4 {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2_g __attribute__((ext_vector_type(2)));

constexpr int kGemmThreads = 256;                 // 4 waves (general path)
constexpr int kTM = 256;                          // tokens per workgroup tile
constexpr int kTN = 256;                          // output features per workgroup tile
// fast path
constexpr int kTK = 128;                          // K per stage (one scale block, whole 128-B lines)
constexpr int kStages = 2;                        // LDS buffers; loads run one stage ahead
constexpr int kStage = (kTM + kTN) * kTK;         // bytes of one LDS stage (64 KB)
constexpr int kFastThreads = 512;                 // 8 waves, two per SIMD
constexpr int kMaxFastBlocks = 56;                // scale blocks staged in LDS (K <= 7168)
// general path
constexpr int kTK1 = 128;
constexpr int kStage1 = (kTM + kTN) * kTK1;       // 64 KB

// s_waitcnt immediate (gfx9 encoding) that waits for vmcnt <= n and nothing else.
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

namespace {

// Token tile `mtile` (in expert order) -> expert, its first row and the tile's rows.
// False if the tile does not exist.  Experts are scanned 64 at a time, one per lane.
__device__ __forceinline__ bool find_tile(const int32_t* __restrict__ offs, int G, uint32_t mtile,
                                          int& g_out, int64_t& row0, int& rows)
{
    const int lane = threadIdx.x & 63;
    uint32_t run = 0;
    for (int g0 = 0; g0 < G; g0 += 64) {
        const int h = g0 + lane;
        const int32_t r0 = h < G ? offs[h] : 0;
        const int32_t mg = h < G ? offs[h + 1] - r0 : 0;
        const uint32_t nt = (uint32_t)(mg + kTM - 1) / kTM;
        uint32_t incl = nt;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const uint32_t o = __shfl_up(incl, d, 64);
            if (lane >= d)
                incl += o;
        }
        const uint32_t first = run + incl - nt;
        const uint64_t mask = __ballot(nt > 0 && mtile >= first && mtile < first + nt);
        if (mask) {
            const int src = __builtin_ctzll(mask);
            const uint32_t j = mtile - (uint32_t)__builtin_amdgcn_readlane((int)first, src);
            const int32_t base = __builtin_amdgcn_readlane(r0, src);
            const int32_t m = __builtin_amdgcn_readlane(mg, src);
            g_out = g0 + src;
            row0 = (int64_t)base + (int64_t)kTM * j;
            rows = min(kTM, m - kTM * (int)j);
            return true;
        }
        run = uniform(run + (uint32_t)__shfl(incl, 63, 64));
    }
    return false;
}

// Workgroup -> (token tile, feature tile).  The tiles of one XCD run in this order:
// groups of kGroupM token tiles, every feature tile of a group before the next group,
// the group's token tiles innermost, so the workgroups one XCD holds at a time share a
// few operand tiles of each kind in its L2.
constexpr uint32_t kGroupM = 4;

// Workgroup -> position in that order for the fast kernel.  Workgroups are dealt
// round-robin over the 8 XCDs; XCD x takes tile groups x, x + 8, x + 16, ... (a group is
// kGroupM token tiles across all feature tiles), so that an XCD's workgroups share a
// group's operand tiles in its L2 while the eight XCDs work on neighbouring groups, that
// is on the same expert's weights at the same time.  The remainder past the last whole
// round of 8 groups keeps its order.
__device__ __forceinline__ uint32_t group_interleave(uint32_t bid, uint32_t nblocks, uint32_t gsz)
{
    const uint32_t round = 8 * gsz;
    const uint32_t full = nblocks / round * round;
    if (bid >= full)
        return bid;
    const uint32_t x = bid & 7, slot = bid >> 3;
    return (x + 8 * (slot / gsz)) * gsz + slot % gsz;
}
__device__ __forceinline__ void tile_of(uint32_t lin, uint32_t nblocks, uint32_t ntn, uint32_t& mtile,
                                        uint32_t& ntile)
{
    const uint32_t ntm = nblocks / ntn;
    const uint32_t grp = lin / (kGroupM * ntn);
    const uint32_t gm = min(kGroupM, ntm - grp * kGroupM);
    const uint32_t idx = lin - grp * kGroupM * ntn;
    mtile = grp * kGroupM + idx % gm;
    ntile = idx / gm;
}

}  // namespace

__global__ __launch_bounds__(kGemmThreads, 1) void fp8_gemm_general_kernel(
    const uint8_t* __restrict__ a, const uint8_t* __restrict__ sa, const uint8_t* __restrict__ w,
    const uint8_t* __restrict__ sw, uint16_t* __restrict__ y, const int32_t* __restrict__ offs, int G,
    int64_t N, int64_t K)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kStage1];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    uint32_t mtile, ntile;
    tile_of(xcd_remap(blockIdx.x, gridDim.x), gridDim.x, (uint32_t)(N / kTN), mtile, ntile);
    int g;
    int64_t row0;
    int rows;
    if (!find_tile(offs, G, mtile, g, row0, rows))
        return;                                   // uniform over the workgroup
    const int64_t n0 = (int64_t)kTN * ntile;
    const uint32_t kb_n = (uint32_t)(K / kTK1);    // scale blocks along K

    // operand tiles: tokens (rows row0 ..) of A and features (rows n0 ..) of W_g
    const __amdgpu_buffer_rsrc_t ra = strip_rsrc(a + row0 * K, (uint64_t)rows * (uint64_t)K);
    const __amdgpu_buffer_rsrc_t rw = strip_rsrc(w + ((int64_t)g * N + n0) * K, (uint64_t)kTN * (uint64_t)K);
    const __amdgpu_buffer_rsrc_t rsa = strip_rsrc(sa + row0 * kb_n, (uint64_t)rows * kb_n);
    const __amdgpu_buffer_rsrc_t rsw = strip_rsrc(sw + ((int64_t)g * N + n0) * kb_n, (uint64_t)kTN * kb_n);

    // loader role: thread t loads chunk c = t & 7 of rows 32 i + (t >> 3), i = 0..7
    const uint32_t lrow = (uint32_t)(tid >> 3), lchunk = (uint32_t)(tid & 7);
    const uint32_t loff = lrow * (uint32_t)K + 16 * lchunk;           // + 32 i K
    const uint32_t lds_w = lrow * kTK1 + 16 * (lchunk ^ ((lrow >> 1) & 7));   // + 32 i kTK1
    // compute role: wave (wm, wn), lane (r, h)
    const int wm = wave & 1, wn = wave >> 1;
    const uint32_t r = (uint32_t)(lane & 31), h = (uint32_t)(lane >> 5);
    const uint32_t sw8 = (r >> 1) & 7;                                 // the swizzle of rows r + 32 x
    // scale byte offsets of the lane's rows (features 128 wn + 32 nt + r, tokens 128 wm + 32 mt + r)
    uint32_t soff_w[4], soff_a[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        soff_w[t] = (uint32_t)(128 * wn + 32 * t + r) * kb_n;
        soff_a[t] = (uint32_t)(128 * wm + 32 * t + r) * kb_n;
    }

    u32x4 ra_reg[8], rw_reg[8];
    auto load_tiles = [&](uint32_t kb) {
        const int koff = (int)(kb * kTK1);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            ra_reg[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                      ra, (int)(loff + 32u * i * (uint32_t)K), koff, 0));
            rw_reg[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                      rw, (int)(loff + 32u * i * (uint32_t)K), koff, 0));
        }
    };
    auto store_tiles = [&](uint32_t stage) {
        uint8_t* const sa_l = lds + stage * kStage1;          // tokens: bytes [0, 32 KB)
        uint8_t* const sw_l = sa_l + kTM * kTK1;              // features: bytes [32 KB, 64 KB)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            *reinterpret_cast<u32x4*>(sa_l + lds_w + 32 * i * kTK1) = ra_reg[i];
            *reinterpret_cast<u32x4*>(sw_l + lds_w + 32 * i * kTK1) = rw_reg[i];
        }
    };
    uint32_t sc_w[4], sc_a[4];                    // current step's scale bytes
    uint32_t nx_w[4], nx_a[4];
    auto load_scales = [&](uint32_t kb, uint32_t (&dw)[4], uint32_t (&da)[4]) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            dw[t] = __builtin_amdgcn_raw_buffer_load_b8(rsw, (int)soff_w[t], (int)kb, 0);
            da[t] = __builtin_amdgcn_raw_buffer_load_b8(rsa, (int)soff_a[t], (int)kb, 0);
        }
    };

    f32x16 acc[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
            acc[mt][nt] = f32x16{};

    load_tiles(0);
    load_scales(0, sc_w, sc_a);
    store_tiles(0);
    __syncthreads();

    for (uint32_t kb = 0; kb < kb_n; ++kb) {
        const uint32_t cur = kb & 1;
        const bool more = kb + 1 < kb_n;
        if (more) {
            load_tiles(kb + 1);
            load_scales(kb + 1, nx_w, nx_a);
        }
        const uint8_t* const ta = lds + cur * kStage1 + (128 * wm) * kTK1;
        const uint8_t* const tw = lds + cur * kStage1 + kTM * kTK1 + (128 * wn) * kTK1;
        __builtin_amdgcn_s_setprio(1);            // matrix work first, as in the fast path
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
            const uint32_t c0 = 16 * ((4 * kh + h) ^ sw8), c1 = 16 * ((4 * kh + 2 + h) ^ sw8);
            i32x8 fw[4], fa[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const uint8_t* const rowp_w = tw + (32 * t + r) * kTK1;
                const uint8_t* const rowp_a = ta + (32 * t + r) * kTK1;
                const u32x4 w0 = *reinterpret_cast<const u32x4*>(rowp_w + c0);
                const u32x4 w1 = *reinterpret_cast<const u32x4*>(rowp_w + c1);
                const u32x4 a0 = *reinterpret_cast<const u32x4*>(rowp_a + c0);
                const u32x4 a1 = *reinterpret_cast<const u32x4*>(rowp_a + c1);
                fw[t] = i32x8{(int)w0.x, (int)w0.y, (int)w0.z, (int)w0.w, (int)w1.x, (int)w1.y, (int)w1.z, (int)w1.w};
                fa[t] = i32x8{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
            }
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int nt = 0; nt < 4; ++nt)
                    acc[mt][nt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        fw[nt], fa[mt], acc[mt][nt], 0, 0, 0, (int)sc_w[nt], 0, (int)sc_a[mt]);
        }
        __builtin_amdgcn_s_setprio(0);
        if (more) {
            store_tiles(cur ^ 1);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                sc_w[t] = nx_w[t];
                sc_a[t] = nx_a[t];
            }
        }
        __syncthreads();
    }

    // epilogue: lane (r, h) of MFMA tile (mt, nt) holds token 128 wm + 32 mt + r and
    // features 128 wn + 32 nt + 8 q + 4 h + (0..3) in values 4q .. 4q + 3
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        const int mloc = 128 * wm + 32 * mt + (int)r;
        if (mloc >= rows)
            continue;
        uint16_t* const yrow = y + (row0 + mloc) * N + n0 + 128 * wn + 4 * h;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x16& v = acc[mt][nt];
                const bf16x2_g p0 = {(__bf16)v[4 * q + 0], (__bf16)v[4 * q + 1]};
                const bf16x2_g p1 = {(__bf16)v[4 * q + 2], (__bf16)v[4 * q + 3]};
                *reinterpret_cast<u32x2*>(yrow + 32 * nt + 8 * q) =
                    u32x2{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1)};
            }
    }
}

// What a wave of the fast kernel needs in its stage loop.
struct FastCtx {
    uint8_t* stage[kStages];                      // the LDS buffers
    const uint8_t* scl_a;                         // staged block scales
    const uint8_t* scl_w;
    __amdgpu_buffer_rsrc_t ra, rw;                // token and feature rows of the tile
    uint32_t loff[4];                             // the lane's loader offsets
    int wave, wm, wn;
    uint32_t r, h;
};

// The LDS loads of stage s into buffer buf: instruction i of wave w fills LDS rows
// 32 w + 8 i .. + 7 of each operand (8 rows x 128 bytes).
__device__ __forceinline__ void fast_issue(const FastCtx& cx, uint32_t s, int buf)
{
    typedef __attribute__((address_space(3))) uint8_t lds_u8;
    const int koff = (int)(s * kTK);
    lds_u8* const st = (lds_u8*)cx.stage[buf];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(cx.ra, st + (32 * cx.wave + 8 * i) * kTK, 16, cx.loff[i], koff, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(cx.rw, st + kTM * kTK + (32 * cx.wave + 8 * i) * kTK, 16,
                                                 cx.loff[i], koff, 0, 0);
    }
}

// The fragments of one MFMA K-step (64 of K) of a wave: two feature tiles, four token tiles.
struct FastFrag {
    i32x8 w[2];
    i32x8 a[4];
};

// A lane's fragment of one operand row for one MFMA K-step: the row's 16-byte LDS chunks
// at byte offsets c0 and c1.
__device__ __forceinline__ i32x8 fast_frag(const uint8_t* rowp, uint32_t c0, uint32_t c1)
{
    const u32x4 v0 = *reinterpret_cast<const u32x4*>(rowp + c0);
    const u32x4 v1 = *reinterpret_cast<const u32x4*>(rowp + c1);
    return i32x8{(int)v0.x, (int)v0.y, (int)v0.z, (int)v0.w, (int)v1.x, (int)v1.y, (int)v1.z, (int)v1.w};
}

// The stage's block scales for the lane's four token tiles and two feature tiles.
__device__ __forceinline__ void fast_scales(const FastCtx& cx, uint32_t t, uint32_t& sca4, uint32_t& scw4)
{
    sca4 = *reinterpret_cast<const uint32_t*>(cx.scl_a + t * kTM + cx.wm * 128 + cx.r * 4);
    // features 64 wn + 32 nt + r are scale row 128 (wn / 2) + 32 (2 (wn % 2) + nt) + r
    scw4 = *reinterpret_cast<const uint32_t*>(cx.scl_w + t * kTN + (cx.wn >> 1) * 128 + cx.r * 4) >>
           (16 * (cx.wn & 1));
}

// The eight MFMAs of one K-step on `cur`.  With kRead, the fragments of K-step j of the
// stage in buffer buf are read into `next` between them (the feature tiles first, then
// one token tile after each token tile's MFMAs), so that a wave's reads overlap its own
// matrix work and the registers of `cur` free up as `next` fills.  The wave with matrix
// work to issue goes first: of a SIMD's two waves, one computes while the other waits.
template <bool kRead>
__device__ __forceinline__ void fast_step(const FastCtx& cx, const FastFrag& cur, uint32_t sca4, uint32_t scw4,
                                          f32x16 (&acc)[4][2], int buf, int j, FastFrag& next)
{
    const uint32_t sw8 = (cx.r >> 1) & 7;                              // the swizzle of rows r + 32 x
    const uint8_t* const ta = cx.stage[buf] + (128 * cx.wm + cx.r) * kTK;
    const uint8_t* const tw = cx.stage[buf] + (kTM + 64 * cx.wn + cx.r) * kTK;
    const uint32_t c0 = 16 * ((4 * j + cx.h) ^ sw8), c1 = 16 * ((4 * j + 2 + cx.h) ^ sw8);
    if (kRead) {
        next.w[0] = fast_frag(tw, c0, c1);
        next.w[1] = fast_frag(tw + 32 * kTK, c0, c1);
    }
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
            acc[mt][nt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                cur.w[nt], cur.a[mt], acc[mt][nt], 0, 0, 0, (int)((scw4 >> (8 * nt)) & 0xFF), 0,
                (int)((sca4 >> (8 * mt)) & 0xFF));
        if (kRead)
            next.a[mt] = fast_frag(ta + 32 * mt * kTK, c0, c1);
    }
    __builtin_amdgcn_s_setprio(0);
}

// Stages t0 (buffer 0) and t0 + 1 (buffer 1), software-pipelined by K-step.  On entry
// f holds the fragments of stage t0's first K-step and (sca, scw) its scales.  Per
// stage t in buffer u: the first K-step's MFMAs issue while the second K-step's
// fragments are read; the lane waits for its loads of stage t + 1 and meets the other
// waves at the barrier (every wave's part of stage t + 1 is then in LDS, and every wave
// has read all of buffer u); stage t + 2 is loaded into buffer u; the second K-step's
// MFMAs issue while the first K-step of stage t + 1 is read.  The barrier thus never
// leaves a wave without matrix work queued behind it.  kLast: t0 + 2 == T.
template <bool kLast>
__device__ __forceinline__ void fast_pair(const FastCtx& cx, uint32_t t0, FastFrag& f, uint32_t& sca,
                                          uint32_t& scw, f32x16 (&acc)[4][2])
{
#pragma unroll
    for (int u = 0; u < kStages; ++u) {
        const uint32_t t = t0 + u;
        FastFrag g;
        fast_step<true>(cx, f, sca, scw, acc, u, 1, g);
        const uint32_t sca_t = sca, scw_t = scw;
        if (!kLast || u == 0) {
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
            __syncthreads();
            if (!kLast)
                fast_issue(cx, t + 2, u);
            fast_scales(cx, t + 1, sca, scw);
            fast_step<true>(cx, g, sca_t, scw_t, acc, u ^ 1, 0, f);
        } else {
            fast_step<false>(cx, g, sca_t, scw_t, acc, 0, 0, f);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

__global__ __launch_bounds__(kFastThreads, 1) void fp8_gemm_kernel(
    const uint8_t* __restrict__ a, const uint8_t* __restrict__ sa, const uint8_t* __restrict__ w,
    const uint8_t* __restrict__ sw, uint16_t* __restrict__ y, const int32_t* __restrict__ offs, int G,
    int64_t N, int64_t K)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds0[kStage];
    __shared__ __attribute__((aligned(16))) uint8_t lds1[kStage];
    // block scales: [block][half][row 0..31][tile 0..3] per operand
    __shared__ __attribute__((aligned(16))) uint8_t scl_a[kMaxFastBlocks * kTM];
    __shared__ __attribute__((aligned(16))) uint8_t scl_w[kMaxFastBlocks * kTN];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    uint32_t mtile, ntile;
    const uint32_t ntn = (uint32_t)(N / kTN);
    tile_of(group_interleave(blockIdx.x, gridDim.x, kGroupM * ntn), gridDim.x, ntn, mtile, ntile);
    int g;
    int64_t row0;
    int rows;
    if (!find_tile(offs, G, mtile, g, row0, rows))
        return;                                   // uniform over the workgroup
    const int64_t n0 = (int64_t)kTN * ntile;
    const uint32_t kb_n = (uint32_t)(K / 128);    // scale blocks along K
    const uint32_t T = (uint32_t)(K / kTK);       // stages

    // operand tiles: tokens (rows row0 ..) of A and features (rows n0 ..) of W_g
    const __amdgpu_buffer_rsrc_t ra = strip_rsrc(a + row0 * K, (uint64_t)rows * (uint64_t)K);
    const __amdgpu_buffer_rsrc_t rw = strip_rsrc(w + ((int64_t)g * N + n0) * K, (uint64_t)kTN * (uint64_t)K);
    const __amdgpu_buffer_rsrc_t rsa = strip_rsrc(sa + row0 * kb_n, (uint64_t)rows * kb_n);
    const __amdgpu_buffer_rsrc_t rsw = strip_rsrc(sw + ((int64_t)g * N + n0) * kb_n, (uint64_t)kTN * kb_n);

    // loader role: instruction i of wave w fills LDS rows 32 w + 8 i .. + 7 of each
    // operand; lane L takes row 32 w + 8 i + L / 8, LDS chunk L % 8, i.e. global chunk
    // (L % 8) ^ ((row >> 1) & 7)
    uint32_t loff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t lrow = (uint32_t)(32 * wave + 8 * i + (lane >> 3));
        loff[i] = lrow * (uint32_t)K + 16 * ((uint32_t)(lane & 7) ^ ((lrow >> 1) & 7));
    }
    // compute role: wave (wm, wn) owns tokens 128 wm .. + 127 and features 64 wn .. + 63;
    // lane (r, h)
    const int wm = wave & 1, wn = wave >> 1;
    const uint32_t r = (uint32_t)(lane & 31), h = (uint32_t)(lane >> 5);
    const FastCtx cx{{lds0, lds1}, scl_a, scl_w, ra, rw, {loff[0], loff[1], loff[2], loff[3]}, wave, wm, wn, r, h};
    // stage the tile's block scales: thread t < 256 owns token row t, thread 256 + t
    // feature row t (row 128 x + 32 q + y goes to byte [block][x][y][q]); rows past the
    // tile read as zero
    {
        const uint32_t t8 = (uint32_t)tid & 255;
        const uint32_t x = t8 >> 7, q = (t8 >> 5) & 3, yy = t8 & 31;
        const uint32_t dst = x * 128 + yy * 4 + q;
        const __amdgpu_buffer_rsrc_t rs = wave < 4 ? rsa : rsw;
        uint8_t* const scl = wave < 4 ? scl_a : scl_w;
        if ((kb_n & 3) == 0) {
            // a row's scale bytes as independent dword loads, all in flight together and
            // with stage 0's operand loads (issued next); dwords past the row's kb_n bytes
            // (the next row's, or zero past the range) land in block slots no stage reads
            uint32_t v4[kMaxFastBlocks / 4];
#pragma unroll
            for (int j = 0; j < kMaxFastBlocks / 4; ++j)
                v4[j] = __builtin_amdgcn_raw_buffer_load_b32(rs, (int)(t8 * kb_n + 4 * j), 0, 0);
            fast_issue(cx, 0, 0);
#pragma unroll
            for (int j = 0; j < kMaxFastBlocks / 4; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    scl[(4 * j + i) * kTM + dst] = (uint8_t)(v4[j] >> (8 * i));
        } else {
            for (uint32_t b = 0; b < kb_n; ++b)
                scl[b * kTM + dst] = (uint8_t)__builtin_amdgcn_raw_buffer_load_b8(rs, (int)(t8 * kb_n + b), 0, 0);
            fast_issue(cx, 0, 0);
        }
    }

    f32x16 acc[4][2];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
            acc[mt][nt] = f32x16{};

    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();                              // scales staged, stage 0 in LDS
    fast_issue(cx, 1, 1);
    FastFrag f;
    uint32_t sca, scw;
    fast_scales(cx, 0, sca, scw);
    {
        const uint32_t sw8 = (cx.r >> 1) & 7;
        const uint8_t* const ta = cx.stage[0] + (128 * cx.wm + cx.r) * kTK;
        const uint8_t* const tw = cx.stage[0] + (kTM + 64 * cx.wn + cx.r) * kTK;
        const uint32_t c0 = 16 * (cx.h ^ sw8), c1 = 16 * ((2 + cx.h) ^ sw8);
        f.w[0] = fast_frag(tw, c0, c1);
        f.w[1] = fast_frag(tw + 32 * kTK, c0, c1);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
            f.a[mt] = fast_frag(ta + 32 * mt * kTK, c0, c1);
    }
    // T is even (K is a multiple of 256 on this path): stages run in pairs, one per LDS
    // buffer; the last pair is peeled so that every load issue in a pair is fixed at
    // compile time and a pair is one basic block
    uint32_t t0 = 0;
    for (; t0 + kStages < T; t0 += kStages)
        fast_pair<false>(cx, t0, f, sca, scw, acc);
    fast_pair<true>(cx, t0, f, sca, scw, acc);

    // epilogue through LDS: lane (r, h) of MFMA tile (mt, nt) holds token 128 wm + 32 mt + r
    // and features 64 wn + 32 nt + 8 q + 4 h + (0..3) in values 4q .. 4q + 3.  The waves
    // write their BF16 results into the stage buffers (tokens 128 wm .. + 127 into
    // buffer wm, 512 bytes per token, the 16-byte chunk c of token row x at chunk
    // c ^ (x % 32), so that neither the writes nor the row reads below conflict), then
    // every lane stores 16-byte pieces of whole rows: one store instruction of a wave
    // covers two 512-byte row segments (four whole 128-byte lines each), where the
    // registers alone would give 32 rows of 16 bytes.  The stores go through a buffer
    // resource whose range is the tile's existing rows, so rows past them are dropped
    // without a branch.
    __syncthreads();                              // every wave is done reading the last stage
    {
        uint8_t* const ob = wm ? lds1 : lds0;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x16& v = acc[mt][nt];
                    const bf16x2_g p0 = {(__bf16)v[4 * q + 0], (__bf16)v[4 * q + 1]};
                    const bf16x2_g p1 = {(__bf16)v[4 * q + 2], (__bf16)v[4 * q + 3]};
                    const uint32_t c = 8 * (uint32_t)wn + 4 * nt + q;
                    *reinterpret_cast<u32x2*>(ob + (32 * mt + r) * 512 + 16 * (c ^ r) + 8 * h) =
                        u32x2{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1)};
                }
    }
    __syncthreads();
    const __amdgpu_buffer_rsrc_t ry = strip_rsrc(y + row0 * N, (uint64_t)rows * (uint64_t)N * 2);
    {
        const uint32_t c = (uint32_t)tid & 31;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint32_t row = ((uint32_t)tid >> 5) + 16 * i;          // tile row 0 .. 255
            const uint8_t* const src = (i < 8 ? lds0 : lds1) + (row & 127) * 512 + 16 * (c ^ (row & 31));
            __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const u32x4*>(src), ry,
                                                   (int)((row * (uint32_t)N + (uint32_t)n0) * 2 + 16 * c), 0,
                                                   2);            // non-temporal: written once
        }
    }
}

int64_t gemm_tile_capacity(int64_t M_cap, int32_t G)
{
    return (M_cap + kTM - 1) / kTM + G;
}

hipError_t launch_fp8_gemm(const uint8_t* a, const uint8_t* sa, const uint8_t* w, const uint8_t* sw,
                           uint16_t* y, const int32_t* offs, int32_t G, int64_t M_cap, int64_t N, int64_t K,
                           hipStream_t stream)
{
    if (M_cap == 0)
        return hipSuccess;
    const int64_t grid = gemm_tile_capacity(M_cap, G) * (N / kTN);
    if (grid > 0x7FFFFFFF)
        return hipErrorInvalidValue;
    int g = G;
    int64_t n = N, k = K;
    void* args[] = {(void*)&a, (void*)&sa, (void*)&w, (void*)&sw, (void*)&y, (void*)&offs, (void*)&g,
                    (void*)&n, (void*)&k};
    const bool fast = K <= 128 * kMaxFastBlocks && K % (kTK * kStages) == 0;
    const void* kern = fast ? (const void*)fp8_gemm_kernel : (const void*)fp8_gemm_general_kernel;
    return launch_kernel(kern, dim3((unsigned)grid), dim3(fast ? kFastThreads : kGemmThreads), args, stream);
}

}  // namespace mxfp4
