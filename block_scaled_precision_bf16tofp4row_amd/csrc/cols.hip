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
//            4rq..4rq+3 of the strip and their MX scale bytes (loaded two strips
//            ahead); four consecutive lanes cover one row's 64 contiguous code bytes
//            and 4 contiguous scale bytes.  The FP8 scale of each (block, group) is a
//            DPP / cross-lane max inside the wave plus an LDS exchange between the
//            block's two waves.  Each row is converted with the gap table of its own
//            scale (even and odd codes separately, one v_perm_b32 each), and 4x4 byte
//            transposes turn 4 rows x 32 columns into 32 dwords (4 rows of one column
//            each), written into a k-major LDS tile: one LDS row per output column k
//            holding that column's strip bytes in output order;
//   stage B  16 lanes per output row: lane c stores the 16-byte aligned chunk c of the
//            strip's output range.  The four rows of one step are 16 columns apart, so
//            their misalignment delta (mod 16) is the same and the realignment is two
//            aligned 16-byte LDS reads plus v_alignbyte_b32 under a wave-uniform
//            branch; every global store is an aligned 16-byte store and 16 lanes cover a
//            contiguous 256-byte
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
constexpr int kLdsBytes = kTileCols * kLdsRowBytes + 64 * 3 + 16;   // + slack for the last row's window
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

// 16 bytes starting `o` bytes into the 32 bytes (lo, hi); o is wave-uniform, so the
// switch is a scalar branch and each output dword is one v_alignbyte_b32.
__device__ __forceinline__ u32x4 window16(const u32x4& lo, const u32x4& hi, uint32_t o)
{
    const uint32_t D[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    const uint32_t v = o & 3;
#define MXFP4_WINDOW(U) \
    u32x4{__builtin_amdgcn_alignbyte(D[U + 1], D[U], v), __builtin_amdgcn_alignbyte(D[U + 2], D[U + 1], v), \
          __builtin_amdgcn_alignbyte(D[U + 3], D[U + 2], v), __builtin_amdgcn_alignbyte(D[U + 4], D[U + 3], v)}
    switch (o >> 2) {
    case 0: return MXFP4_WINDOW(0);
    case 1: return MXFP4_WINDOW(1);
    case 2: return MXFP4_WINDOW(2);
    default: return MXFP4_WINDOW(3);
    }
#undef MXFP4_WINDOW
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
    int64_t r_lo;              // the strip's first row, relative to row0
    int nrows;                 // rows in the strip
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
            r.r_lo = (int64_t)(s - r.sb) * kStripRows;
            r.nrows = (int)min<int64_t>(kStripRows, r.mg - r.r_lo);
            return r;
        }
        run_s += t.total_s;
        run_b += t.total_b;
    }
}

// Info of strip s, reusing `prev` (an earlier strip) when s is in the same expert.
__device__ __forceinline__ StripInfo strip_after(const int32_t* __restrict__ offs, int G,
                                                 const ExpertTable& cached, const StripInfo& prev,
                                                 uint32_t s)
{
    if (s < prev.sb + (uint32_t)((prev.mg + kStripRows - 1) / kStripRows)) {
        StripInfo r = prev;
        r.r_lo = (int64_t)(s - r.sb) * kStripRows;
        r.nrows = (int)min<int64_t>(kStripRows, r.mg - r.r_lo);
        return r;
    }
    return locate(offs, G, cached, s);
}

// ---- the kernel ---------------------------------------------------------------------------

struct RowsIn {
    u32x4 c[4];                // codes of group kc, rows 4rq..4rq+3
    uint32_t s[4];             // their MX scale bytes (0 for rows past the strip)
};

// Loads are unconditional (rows past the strip are clamped to its last row and zeroed
// after the load), so every strip issues the same straight-line sequence of loads and the
// compiler can wait for exactly the loads it needs.
__device__ __forceinline__ RowsIn load_rows(const uint8_t* __restrict__ codes,
                                            const uint8_t* __restrict__ scales, int64_t K,
                                            int64_t row_first, int nrows, int rq, int kc,
                                            uint32_t kt)
{
    RowsIn in;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = min(4 * rq + i, nrows - 1);
        const int64_t row = row_first + r;
        in.c[i] = *reinterpret_cast<const u32x4*>(codes + row * (K / 2) + 64 * (int64_t)kt + 16 * kc);
        in.s[i] = scales[row * (K / 32) + 4 * (int64_t)kt + kc];
    }
    return in;
}

__device__ __forceinline__ void mask_rows(RowsIn& in, int nrows, int rq)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const bool ok = 4 * rq + i < nrows;
        in.c[i] = ok ? in.c[i] : u32x4{0, 0, 0, 0};
        in.s[i] = ok ? in.s[i] : 0u;
    }
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
    // stage B: wave (half hb, parity pb) converts output rows 64hb + 8pb + it + 16q
    // (it = 0..7 steps, q = lane >> 4): rows 16 apart share their misalignment mod 16
    const int hb = wave >> 1, pb = wave & 1;
    const uint32_t kb0 = 64 * hb + 8 * pb + 16 * (lane >> 4);              // row at it = 0


    // one strip is converted while the next one is loaded; the loop is unrolled by two
    // so the two register sets alternate roles without copies
    auto convert_strip = [&](const StripInfo& cur, RowsIn in, bool carry_in, bool carry_out) {
        const int64_t r_lo = cur.r_lo;
        const int nrows = cur.nrows;
        mask_rows(in, nrows, rq);

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
        // writes from align128(A), and when the next strip continues the row it stops at
        // the last line boundary, leaving the rest in the carry area.  So in the steady
        // state every store belongs to a whole 128-byte line (16 lanes x 16 bytes = two
        // lines per row).  Memory byte b of the row maps to LDS row byte kData + (b - A);
        // since b is 16-aligned, the offset inside the aligned LDS chunk is
        // o = (16 - (A & 15)) & 15 for every chunk of the four rows of a step.
        int64_t A = K * cur.row0 + (kTileCols * (int64_t)kt + kb0) * cur.mg + r_lo;
        const bool steady = carry_in && carry_out;
#pragma unroll 2
        for (int it = 0; it < 8; ++it, A += cur.mg) {
            const uint32_t kl = kb0 + it;
            const uint8_t* rowp = tile + lds_row(kl) + kData;          // LDS byte of strip byte 0
            const uint32_t o = __builtin_amdgcn_readfirstlane((uint32_t)(16 - (A & 15)) & 15);
            if (steady) {
                const int64_t b0 = (A & ~(int64_t)127) + 16 * c;       // two whole lines
                const uint8_t* src = rowp + (b0 - A) - o;              // 16-byte aligned
                const u32x4 lo = *reinterpret_cast<const u32x4*>(src);
                u32x4 v = lo;
                if (o != 0)
                    v = window16(lo, *reinterpret_cast<const u32x4*>(src + 16), o);
                *reinterpret_cast<u32x4*>(yT + b0) = v;
            } else {
                const int64_t E = A + nrows;
                const int64_t W_lo = carry_in ? (A & ~(int64_t)127) : A;
                const int64_t W_hi = carry_out ? (E & ~(int64_t)127) : E;
                const int64_t j0 = W_lo >> 4;                          // first 16-byte chunk
                const int nch = W_hi > W_lo ? (int)(((W_hi + 15) >> 4) - j0) : 0;
                for (int pass = 0; pass < 2; ++pass) {
                    const int jj = c + 16 * pass;
                    if (jj >= nch)
                        continue;
                    const int64_t b0 = (j0 + jj) << 4;
                    const uint8_t* src = rowp + (b0 - A) - o;
                    const u32x4 lo = *reinterpret_cast<const u32x4*>(src);
                    u32x4 v = lo;
                    if (o != 0)
                        v = window16(lo, *reinterpret_cast<const u32x4*>(src + 16), o);
                    if (b0 >= W_lo && b0 + 16 <= W_hi) {
                        *reinterpret_cast<u32x4*>(yT + b0) = v;
                    } else {
                        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
                        for (int q = 0; q < 16; ++q)
                            if (b0 + q >= W_lo && b0 + q < W_hi)
                                yT[b0 + q] = (uint8_t)(w4[q >> 2] >> (8 * (q & 3)));
                    }
                }
            }
        }
        // the next strip continues these rows: move the last 128 strip bytes of each of
        // this wave's 32 rows into the carry area (only this wave reads these rows)
        if (carry_out) {
            const int r = lane >> 1;                                   // 0..31
            uint8_t* row = tile + lds_row(64 * hb + 8 * pb + (r & 7) + 16 * (r >> 3)) + 64 * (lane & 1);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                *reinterpret_cast<u32x4*>(row + 16 + 16 * q) =
                    *reinterpret_cast<const u32x4*>(row + kData + kStripRows - kCarryBytes + 16 * q);
        }

    };

    StripInfo info = locate(offs, G, t0, s0);
    RowsIn inA = load_rows(codes, scales, K, info.row0 + info.r_lo, info.nrows, rq, kc, kt);
    RowsIn inB;
    bool carry = false;                           // LDS carry areas hold the previous strip's tail
    for (uint32_t s = s0; s < s1; s += 2) {
        // strip s (registers A); load strip s + 1 (registers B) meanwhile
        const bool has1 = s + 1 < s1;
        const StripInfo info1 = has1 ? strip_after(offs, G, t0, info, s + 1) : info;
        inB = load_rows(codes, scales, K, info1.row0 + info1.r_lo, info1.nrows, rq, kc, kt);
        const bool c1 = has1 && info1.sb == info.sb;
        convert_strip(info, inA, carry, c1);
        if (!has1)
            break;
        // strip s + 1 (registers B); load strip s + 2 (registers A) meanwhile
        const bool has2 = s + 2 < s1;
        const StripInfo info2 = has2 ? strip_after(offs, G, t0, info1, s + 2) : info1;
        inA = load_rows(codes, scales, K, info2.row0 + info2.r_lo, info2.nrows, rq, kc, kt);
        const bool c2 = has2 && info2.sb == info1.sb;
        convert_strip(info1, inB, c1, c2);
        info = info2;
        carry = c2;
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
