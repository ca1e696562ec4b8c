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
// Work: a strip is up to 256 consecutive rows (two FP8 blocks) of one expert; each
// expert's rows are cut into strips and all strips are numbered in expert order.
// The grid is persistent: each workgroup owns one 128-column tile (four MX groups)
// and a contiguous range of strips, which it converts in order.
//   stage A  thread (kc = lane & 3, rq) holds the 16 code bytes of group kc for rows
//            4rq..4rq+3 of the strip and their MX scale bytes (loaded one strip
//            ahead); four consecutive lanes cover one row's 64 contiguous code bytes
//            and 4 contiguous scale bytes.  The FP8 scale of each (block, group) is a
//            DPP / cross-lane max inside the wave plus an LDS exchange between the
//            block's two waves.  Each row is converted with the gap table of its own
//            scale (even and odd codes separately, one v_perm_b32 each), and 4x4 byte
//            transposes turn 4 rows x 32 columns into 32 dwords (4 rows of one column
//            each), written into a k-major LDS tile: one LDS row per output column k
//            holding that column's strip bytes in output order;
//   stage B  16 lanes per output row: lane c stores the 16-byte aligned chunk c of the
//            strip's output range.  The range's misalignment delta (the same for every
//            strip of an expert) becomes an unaligned 16-byte LDS read, so every global
//            store is an aligned 16-byte store and 16 lanes cover a contiguous 256-byte
//            run.  A row's stores advance on 128-byte line boundaries: the bytes past
//            a strip's last line boundary are carried in LDS and written with the next
//            strip, so in the steady state every store belongs to a whole 128-byte line
//            (partial lines cost the memory system a read-modify-write).  Only at the
//            ends of a workgroup's run inside an expert are partial lines written.
// LDS skew: the tile row of column k starts at byte 400k + 64 (k >> 5); 32 rows of 400
// bytes span a whole number of bank cycles, so the 64-byte shift per MX group puts the
// stage-A dword writes of the four groups (16 rows each per wave) in 64 distinct banks.
// This plays the role of the page's padded, skewed shared-memory layout.
#include "common.h"

namespace mxfp4 {

__constant__ GapLut kColsGapLut = make_gap_lut();

constexpr int kTileRows = 128;                        // FP8 block along the tokens
constexpr int kTileCols = 128;                        // four MX groups
constexpr int kStripRows = 256;                       // two FP8 blocks
// LDS row of one output column: 16 bytes of slack, a 128-byte carry area holding the
// previous strip's bytes past the last 128-byte line boundary, then the strip's bytes.
constexpr int kCarryBytes = 128;
constexpr int kData = 16 + kCarryBytes;               // strip byte 0 of an LDS row
constexpr int kLdsRowBytes = kData + kStripRows;
constexpr int kLdsBytes = kTileCols * kLdsRowBytes + 64 * 3;
constexpr int kWgPerCu = 3;                           // LDS-limited residency
static_assert(kStripRows == 4 * 64, "stage A maps 64 quads of rows over the 4 waves");
static_assert((32 * (kLdsRowBytes / 4)) % 64 == 0, "32 tile rows must span a multiple of 64 banks");

__device__ __forceinline__ uint32_t lds_row(uint32_t k) { return kLdsRowBytes * k + 64 * (k >> 5); }

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

// ---- strips of experts ----------------------------------------------------------------

// Per-lane expert table for experts 64*chunk + lane: first strip, first 128-row block,
// first row and row count.  Every wave builds it on its own (no barrier).
struct ExpertTable {
    uint32_t sb, bb, ns;       // first strip, first block, strip count (lane's expert)
    int32_t row0, mg;          // first row, rows
    uint32_t total_s, total_b; // strips / blocks of the whole chunk
};

__device__ __forceinline__ ExpertTable expert_chunk(const int32_t* __restrict__ offs, int G, int g0,
                                                    uint32_t run_s, uint32_t run_b)
{
    const int lane = threadIdx.x & 63;
    const int h = g0 + lane;
    ExpertTable t;
    t.row0 = h < G ? offs[h] : 0;
    t.mg = h < G ? offs[h + 1] - t.row0 : 0;
    t.ns = (uint32_t)(t.mg + kStripRows - 1) / kStripRows;
    const uint32_t nb = (uint32_t)(t.mg + kTileRows - 1) / kTileRows;
    uint32_t is = t.ns, ib = nb;
#pragma unroll
    for (int dlt = 1; dlt < 64; dlt <<= 1) {
        uint32_t os = __shfl_up(is, dlt, 64), ob = __shfl_up(ib, dlt, 64);
        if (lane >= dlt) {
            is += os;
            ib += ob;
        }
    }
    t.sb = run_s + is - t.ns;
    t.bb = run_b + ib - nb;
    t.total_s = __shfl(is, 63, 64);
    t.total_b = __shfl(ib, 63, 64);
    return t;
}

struct StripInfo {
    int64_t row0, mg;          // expert's first row and row count
    uint32_t sb, bb;           // expert's first strip and first 128-row block
};

// Expert of global strip s (s < total strips).  `cached` is the table of experts
// 0..63, used directly when G <= 64; larger G rescans 64 experts at a time.
__device__ __forceinline__ StripInfo locate(const int32_t* __restrict__ offs, int G,
                                            const ExpertTable& cached, uint32_t s)
{
    ExpertTable t = cached;
    uint32_t run_s = 0, run_b = 0;
    for (int g0 = 0;; g0 += 64) {
        if (g0 > 0)
            t = expert_chunk(offs, G, g0, run_s, run_b);
        const bool mine = t.ns > 0 && s >= t.sb && s < t.sb + t.ns;
        const uint64_t mask = __ballot(mine);
        if (mask || g0 + 64 >= G) {
            const int src = mask ? __builtin_ctzll(mask) : 0;
            StripInfo r;
            r.row0 = __builtin_amdgcn_readlane(t.row0, src);
            r.mg = __builtin_amdgcn_readlane(t.mg, src);
            r.sb = __builtin_amdgcn_readlane(t.sb, src);
            r.bb = __builtin_amdgcn_readlane(t.bb, src);
            return r;
        }
        run_s += t.total_s;
        run_b += t.total_b;
    }
}

// ---- the kernel ---------------------------------------------------------------------------

struct RowsIn {
    u32x4 c[4];                // codes of group kc, rows 4rq..4rq+3
    uint32_t s[4];             // their MX scale bytes (0 for rows past the strip)
};

__device__ __forceinline__ RowsIn load_rows(const uint8_t* __restrict__ codes,
                                            const uint8_t* __restrict__ scales, int64_t K,
                                            int64_t row_first, int nrows, int rq, int kc,
                                            uint32_t kt)
{
    RowsIn in;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const bool ok = 4 * rq + i < nrows;
        const int64_t row = row_first + 4 * rq + i;
        in.c[i] = ok ? *reinterpret_cast<const u32x4*>(codes + row * (K / 2) + 64 * (int64_t)kt + 16 * kc)
                     : u32x4{0, 0, 0, 0};
        in.s[i] = ok ? (uint32_t)scales[row * (K / 32) + 4 * (int64_t)kt + kc] : 0u;
    }
    return in;
}

__global__ __launch_bounds__(kThreads) void fp8_cols_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    uint8_t* __restrict__ yT, uint8_t* __restrict__ yT_scales,
    const int32_t* __restrict__ offs, int G, int64_t K, int parts)
{
    __shared__ __attribute__((aligned(16))) uint8_t tile[kLdsBytes];
    __shared__ uint32_t wave_max[4];
    __shared__ uint32_t lut[2 * (kMaxGap + 1)];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
    const uint32_t nkt = (uint32_t)(K / kTileCols);
    const uint32_t lambda = xcd_remap(blockIdx.x, gridDim.x);
    const uint32_t kt = lambda % nkt;
    const uint32_t part = lambda / nkt;

    if (tid < 2 * (kMaxGap + 1))
        lut[tid] = kColsGapLut.w[tid >> 1][tid & 1];

    // strips of all experts; this workgroup takes strips [s0, s1) of column tile kt
    const ExpertTable t0 = expert_chunk(offs, G, 0, 0, 0);
    uint32_t n_strips = t0.total_s;
    {
        uint32_t run_s = t0.total_s, run_b = t0.total_b;
        for (int g0 = 64; g0 < G; g0 += 64) {
            const ExpertTable t = expert_chunk(offs, G, g0, run_s, run_b);
            run_s += t.total_s;
            run_b += t.total_b;
        }
        n_strips = run_s;
    }
    const uint32_t s0 = (uint32_t)(((uint64_t)n_strips * part) / (uint32_t)parts);
    const uint32_t s1 = (uint32_t)(((uint64_t)n_strips * (part + 1)) / (uint32_t)parts);
    if (s0 >= s1)
        return;                                   // uniform over the workgroup

    const int kc = lane & 3;                      // MX group inside the tile
    const int rq = (lane >> 2) + 16 * wave;       // rows 4rq..4rq+3 of the strip
    const int c = lane & 15;                      // stage B chunk
    const uint32_t wbase = lds_row(32 * kc) + kData + 4 * rq;              // stage A writes
    const uint32_t rbase = lds_row(32 * wave + (lane >> 4)) + kData;       // stage B rows

    StripInfo cur = locate(offs, G, t0, s0);
    int64_t r_lo = (int64_t)(s0 - cur.sb) * kStripRows;
    int nrows = (int)min<int64_t>(kStripRows, cur.mg - r_lo);
    RowsIn in = load_rows(codes, scales, K, cur.row0 + r_lo, nrows, rq, kc, kt);
    bool carry_in = false;                        // LDS row fronts hold the previous strip's tail

    for (uint32_t s = s0; s < s1; ++s) {
        // ---- next strip: where, and prefetch its rows --------------------------------------
        const bool has_next = s + 1 < s1;
        StripInfo nxt = cur;
        int64_t r_lo_n = r_lo + kStripRows;
        if (has_next && s + 1 >= cur.sb + (uint32_t)((cur.mg + kStripRows - 1) / kStripRows)) {
            nxt = locate(offs, G, t0, s + 1);
            r_lo_n = (int64_t)(s + 1 - nxt.sb) * kStripRows;
        }
        const int nrows_n = has_next ? (int)min<int64_t>(kStripRows, nxt.mg - r_lo_n) : 0;
        const bool carry_out = has_next && nxt.sb == cur.sb;    // next strip continues this expert
        RowsIn nin;
        if (has_next)
            nin = load_rows(codes, scales, K, nxt.row0 + r_lo_n, nrows_n, rq, kc, kt);

        // ---- stage A: block scales ---------------------------------------------------------
        uint32_t m = max(max(in.s[0], in.s[1]), max(in.s[2], in.s[3]));
        m = max(m, (uint32_t)__builtin_amdgcn_update_dpp((int)m, (int)m, 0x124, 0xF, 0xF, false)); // row_ror:4
        m = max(m, (uint32_t)__builtin_amdgcn_update_dpp((int)m, (int)m, 0x128, 0xF, 0xF, false)); // row_ror:8
        m = max(m, (uint32_t)__shfl_xor((int)m, 16, 64));
        m = max(m, (uint32_t)__shfl_xor((int)m, 32, 64));
        const uint32_t packed = __builtin_amdgcn_readlane(m, 0) | (__builtin_amdgcn_readlane(m, 1) << 8) |
                                (__builtin_amdgcn_readlane(m, 2) << 16) | (__builtin_amdgcn_readlane(m, 3) << 24);
        if (lane == 0)
            wave_max[wave] = packed;
        __syncthreads();              // (1) wave maxima visible; every wave is past stage B
        const uint32_t bmax = __builtin_amdgcn_readfirstlane(
            __builtin_bit_cast(uint32_t, __builtin_elementwise_max(
                __builtin_bit_cast(u8x4, wave_max[wave & 2]), __builtin_bit_cast(u8x4, wave_max[(wave & 2) + 1]))));
        const uint32_t S = (bmax >> (8 * kc)) & 0xFF;
        if (tid < 16) {               // block scales: 2 blocks x 128 columns
            const int blk = tid >> 3, piece = tid & 7;
            if (kTileRows * blk < nrows) {
                const uint32_t both = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(
                    __builtin_bit_cast(u8x4, wave_max[2 * blk]), __builtin_bit_cast(u8x4, wave_max[2 * blk + 1])));
                const uint32_t w4 = ((both >> (8 * (piece >> 1))) & 0xFF) * 0x01010101u;
                *reinterpret_cast<u32x4*>(yT_scales + K * (int64_t)(cur.bb + r_lo / kTileRows + blk) +
                                          kTileCols * (int64_t)kt + 16 * piece) = u32x4{w4, w4, w4, w4};
            }
        }

        // ---- stage A: convert, transpose, k-major into LDS ------------------------------
        uint32_t E[4][4], O[4][4];    // [row][code dword]: even / odd codes of 8 columns
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t d = min(S - in.s[i], (uint32_t)kMaxGap);
            const uint32_t lo = lut[2 * d], hi = lut[2 * d + 1];
            convert8_split(in.c[i].x, lo, hi, E[i][0], O[i][0]);
            convert8_split(in.c[i].y, lo, hi, E[i][1], O[i][1]);
            convert8_split(in.c[i].z, lo, hi, E[i][2], O[i][2]);
            convert8_split(in.c[i].w, lo, hi, E[i][3], O[i][3]);
        }
        // code dword q covers columns 8q..8q+7 of the group: even codes -> columns 8q+2m,
        // odd codes -> 8q+2m+1; each transposed dword holds rows 4rq..4rq+3 of a column
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint32_t e[4], o[4];
            transpose4x4(E[0][q], E[1][q], E[2][q], E[3][q], e[0], e[1], e[2], e[3]);
            transpose4x4(O[0][q], O[1][q], O[2][q], O[3][q], o[0], o[1], o[2], o[3]);
#pragma unroll
            for (int mm = 0; mm < 4; ++mm) {
                *reinterpret_cast<uint32_t*>(tile + wbase + kLdsRowBytes * (8 * q + 2 * mm)) = e[mm];
                *reinterpret_cast<uint32_t*>(tile + wbase + kLdsRowBytes * (8 * q + 2 * mm + 1)) = o[mm];
            }
        }
        __syncthreads();              // (2) tile complete

        // ---- stage B: 16 lanes per output row, 4 rows per step, 32 rows per wave ---------
        // Output row k of expert g starts at byte K*offs[g] + k*M_g; this strip's bytes
        // are [A, A + nrows) with A = that + r_lo.  A row's stores advance a frontier on
        // 128-byte line boundaries: with the previous strip's tail carried in, this strip
        // writes [align128(A), ...), and when the next strip continues the row it stops
        // at the last line boundary, leaving the rest in the carry area.  So in the steady
        // state every store is part of a whole 128-byte line (16 lanes x 16 bytes = two
        // lines per row).  Bytes of the written range map to LDS row byte kData + (b - A).
        int64_t A = K * cur.row0 + (kTileCols * (int64_t)kt + 32 * wave + (lane >> 4)) * cur.mg + r_lo;
        const int64_t dA = 4 * cur.mg;
        const bool edges = !(carry_in && carry_out);       // some range ends are not line-aligned
#pragma unroll 2
        for (int it = 0; it < 8; ++it, A += dA) {
            const int64_t E = A + nrows;
            const int64_t W_lo = carry_in ? (A & ~(int64_t)127) : A;
            const int64_t W_hi = carry_out ? (E & ~(int64_t)127) : E;
            const uint8_t* rowp = tile + rbase + kLdsRowBytes * 4 * it;   // LDS byte of strip byte 0
            const int64_t j0 = W_lo >> 4;                     // first 16-byte chunk touched
            const int nch = W_hi > W_lo ? (int)(((W_hi + 15) >> 4) - j0) : 0;
            for (int jj = c; jj < nch; jj += 16) {
                const int64_t b0 = (j0 + jj) << 4;            // chunk start byte
                if (!edges || (b0 >= W_lo && b0 + 16 <= W_hi)) {
                    *reinterpret_cast<u32x4*>(yT + b0) =
                        *reinterpret_cast<const u32x4_unaligned*>(rowp + (b0 - A));
                } else {
                    const int64_t lo = max(b0, W_lo), hi = min(b0 + 16, W_hi);
                    for (int64_t q = lo; q < hi; ++q)
                        yT[q] = rowp[q - A];
                }
            }
        }
        // the next strip continues these rows: move the last 128 strip bytes of each of
        // this wave's 32 rows into the carry area (only this wave reads these rows)
        if (carry_out) {
            uint8_t* row = tile + lds_row(32 * wave + (lane >> 1)) + 64 * (lane & 1);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                *reinterpret_cast<u32x4*>(row + 16 + 16 * q) =
                    *reinterpret_cast<const u32x4*>(row + kData + kStripRows - kCarryBytes + 16 * q);
        }

        carry_in = carry_out;
        cur = nxt;
        r_lo = r_lo_n;
        nrows = nrows_n;
        in = nin;
    }
}

int64_t cols_block_capacity(int64_t M_cap, int32_t G)
{
    return (M_cap + kTileRows - 1) / kTileRows + G;
}

static int device_cus()
{
    static int cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

hipError_t launch_fp8_cols(const uint8_t* codes, const uint8_t* scales, uint8_t* yT,
                           uint8_t* yT_scales, const int32_t* offs, int32_t G, int64_t M_cap,
                           int64_t K, hipStream_t stream)
{
    if (M_cap == 0)
        return hipSuccess;
    const int64_t nkt = K / kTileCols;
    // one resident wave of workgroups: parts per column tile so that nkt * parts fills the
    // GPU, but never more parts than the capacity in strips
    const int64_t cap_strips = (M_cap + kStripRows - 1) / kStripRows + G;
    int64_t parts = (int64_t)device_cus() * kWgPerCu / nkt;
    parts = parts < 1 ? 1 : parts;
    parts = parts > cap_strips ? cap_strips : parts;
    const int64_t grid = nkt * parts;
    if (grid > 0x7FFFFFFF)
        return hipErrorInvalidValue;
    int g = G;
    int64_t k = K;
    int p = (int)parts;
    void* args[] = {(void*)&codes, (void*)&scales, (void*)&yT, (void*)&yT_scales, (void*)&offs,
                    (void*)&g, (void*)&k, (void*)&p};
    return hipLaunchKernel((const void*)fp8_cols_kernel, dim3((unsigned)grid), dim3(kThreads), args,
                           0, stream);
}

}  // namespace mxfp4
