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
// Work: a strip is one 128-row block of one expert; the strips of all experts are
// numbered in expert order (strip s is row s of the block-scale output).  The grid
// is persistent, one workgroup per compute unit: each owns a 256-column tile (eight
// MX groups, so every row it reads is one whole 128-byte line of codes) and a
// contiguous range of strips (every parts-th strip instead when all experts are
// multiples of 4096 rows and no strip carries into the next: strips.h, kDealRows).
// Its sixteen waves have two roles, so that no wave both
// loads and stores (a wave's loads and stores share one in-order completion counter,
// and waiting for a load must not wait for older stores):
//   producers (waves 0-3)   wave w converts rows 32w..32w+31 of every strip: lane
//            (rq = lane >> 3, c = lane & 7) holds the 16 code bytes of group c for
//            rows 32w + 4rq .. + 3, loaded two strips ahead.  The block scale of a
//            group is the max over the strip's 128 rows: each wave reduces its 32
//            rows (a DPP row rotation and the 16- and 32-lane swaps) and publishes
//            the partial max in LDS, and every wave takes the max of the four.  Each row is converted with the
//            gap table of its own scale; 4x4 byte transposes turn 4 rows x 32 columns
//            into 32 dwords (4 rows of one column each), written into a k-major LDS
//            ring: one ring per output column k holding the column's bytes of the
//            last four strips in order;
//   consumers (waves 4-15)  write the output lines of the strip before: 8 lanes per
//            output column, lane c stores bytes [16c, 16c + 16) of the column's
//            128-byte line, 8 columns per instruction, 32 instructions per strip
//            spread over the twelve waves (more storing waves keep more stores in
//            flight; twelve fit beside the producers in 128 VGPRs per lane).  The
//            8 columns of an instruction are 16 apart, so their misalignment (mod 16)
//            is the same (wave-uniform) and the realignment is five dword LDS reads
//            plus four v_alignbyte_b32, with no branch.  A column's stores advance on 128-byte line boundaries: the
//            bytes past a strip's last line boundary stay in the ring and go out with
//            the next strip, so in the steady state every store covers whole
//            128-byte lines (a partial line costs the memory system a read-modify-
//            write).  Only at the ends of a workgroup's run inside an expert are
//            partial lines written.  The output is written once and never re-read
//            here, so the stores are streaming (non-temporal).
// Synchronisation is by monotonic counters in LDS (no barrier inside the strip loop):
// the producers count strips converted and partial maxima published, the consumers
// count per ring slot the strips drained; every wait is bounded (a wave that waits
// about a second gives up and leaves the kernel instead of hanging).
// LDS layout: column k's ring (512 bytes, with its first 32 bytes repeated after it so
// a 32-byte read window never wraps) starts at byte 544k + 32 (k >> 5).  This plays the
// role of the page's padded, skewed shared-memory layout against bank conflicts.
#include "strips.h"

namespace mxfp4 {

constexpr int kProducerWaves = 4;
constexpr int kConsumerWaves = 12;
// a strip is 32 store instructions (256 columns x 128 bytes); consumer wave v issues
// instructions v, v + 12, v + 24 (< 32)
constexpr int kPrefetch = 2;                      // strips of loads in flight per producer wave
constexpr int kColsThreads = 64 * (kProducerWaves + kConsumerWaves);
static_assert(kStripRows == 32 * kProducerWaves, "a producer wave converts 32 rows");
static_assert(kTileCols == 32 * 8, "a producer lane converts one MX group of 8");
static_assert((kRing & (kRing - 1)) == 0, "the ring position wraps with a mask");

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

// ---- producers ---------------------------------------------------------------------------

// A lane's four rows of a strip: eight consecutive lanes read one row's whole 128-byte
// line of codes, so a load instruction touches 8 lines.  Scales are loaded as whole
// dwords (a byte load would be zero-extended where the loop carries it, which makes the
// compiler wait for the prefetched loads early); the byte is extracted at use.  Loads go
// through strip_rsrc (strips.h): rows past a partial strip read as zero codes with scale
// byte 0, which leaves the block scale unchanged; their bytes are never written out.
// Lane offsets within a strip fit in 32 bits (128 rows x K/2 bytes with K <= 2^24).
struct Codes {
    u32x4 c[4];                // 32 codes of the lane's group for each of its four rows
};
struct Scales {
    uint32_t s;                // lane L: dword L & 1 of the 8 scale bytes of wave row L >> 1
};

__device__ __forceinline__ Codes load_codes(const uint8_t* __restrict__ codes, int64_t K,
                                            const StripInfo& st, uint32_t kt, const uint32_t (&off)[4])
{
    Codes in;
    const __amdgpu_buffer_rsrc_t rsrc = strip_rsrc(codes + (st.row0 + st.r_lo) * (K / 2) + 128 * (int64_t)kt,
                                                   (uint64_t)st.nrows * (uint64_t)(K / 2));
#pragma unroll
    for (int i = 0; i < 4; ++i)
        in.c[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)off[i], 0, 0));
    return in;
}

// The 8 scale bytes (groups 0..7 of the tile) of the wave's 32 rows: one dword per lane,
// a single load instruction per strip; lanes fetch their own rows' bytes with
// ds_bpermute at use.  The narrow last tile has groups 0..3 only (one dword per row).
__device__ __forceinline__ Scales load_scales(const uint8_t* __restrict__ scales, int64_t K,
                                              const StripInfo& st, uint32_t kt, uint32_t off)
{
    Scales in;
    const __amdgpu_buffer_rsrc_t rsrc = strip_rsrc(scales + (st.row0 + st.r_lo) * (K / 32) + 8 * (int64_t)kt,
                                                   (uint64_t)st.nrows * (uint64_t)(K / 32));
    in.s = __builtin_amdgcn_raw_buffer_load_b32(rsrc, (int)off, 0, 0);
    return in;
}

// ---- the kernel ---------------------------------------------------------------------------

__global__ __launch_bounds__(kColsThreads, 1) void fp8_cols_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    uint8_t* __restrict__ yT, uint8_t* __restrict__ yT_scales,
    const int32_t* __restrict__ offs, int G, int64_t K, int parts, WaitCtl wc)
{
    __shared__ __attribute__((aligned(16))) uint8_t tile[kTileBytes];
    __shared__ __attribute__((aligned(16))) SlotInfo info[kSlots];
    __shared__ __attribute__((aligned(16))) uint32_t lut[2 * (kMaxGap + 1)];
    // per ring slot, per MX group: the max MX scale byte over each producer wave's 32 rows
    __shared__ __attribute__((aligned(16))) uint32_t pmax[kSlots][8];
    // progress: strips written by producer waves, partial maxima published by producer
    // waves, and per ring slot the strips drained by consumer waves (all monotonic)
    __shared__ uint32_t produced, published, drained[kSlots];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
    const uint32_t nkt = (uint32_t)((K + kTileCols - 1) / kTileCols);
    const uint32_t lambda = xcd_remap(blockIdx.x, gridDim.x);
    const uint32_t kt = lambda % nkt;
    const uint32_t part = lambda / nkt;
    // the last tile is 128 columns wide when K is an odd multiple of 128
    const int ncols = (int)min<int64_t>(kTileCols, K - (int64_t)kTileCols * kt);

    // this workgroup's strips of column tile kt (strip_run, strips.h): a contiguous range,
    // with a lead-in strip where it starts inside an expert, or every parts-th strip of
    // a segment whose strips are independent
    const ExpertTable t0 = expert_chunk(offs, G, 0, 0);
    StripRun run;
    if (!strip_run(offs, G, t0, part, (uint32_t)parts, run))
        return;                                   // uniform over the workgroup
    const uint32_t n = run.n;                     // strips this workgroup converts

    // Producer lanes (waves 0 .. kProducerWaves - 1): wave w converts rows 32w..32w+31 of
    // each strip; lane (rq, c) holds group c (tile columns 32c..32c+31) of rows
    // 32w + 4rq .. + 3.  Their first kPrefetch strips' loads go out before the barrier,
    // so they travel while the table and counters are set.
    const int c = lane & 7;
    const int rq = lane >> 3;
    const int row_q = 32 * wave + 4 * rq;         // first of the lane's four rows
    // the narrow last tile has groups 0..3: lanes of groups 4..7 repeat group c - 4
    // (their columns are never written out)
    const uint32_t cl = 32 * c < ncols ? (uint32_t)c : (uint32_t)(c & 3);
    const uint32_t cbyte = 16 * cl;
    const uint32_t sshift = 8 * (cl & 3);
    // byte offsets within a strip of the lane's four code chunks and of its scale dword
    uint32_t coff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        coff[i] = (uint32_t)(row_q + i) * (uint32_t)(K / 2) + cbyte;
    const uint32_t soff = (uint32_t)(32 * wave + (lane >> 1)) * (uint32_t)(K / 32) +
                          4 * (ncols <= 128 ? 0u : (uint32_t)(lane & 1));
    // Loads run kPrefetch strips ahead of the conversion (repeats of the last strip past
    // the range, so the load sequence never varies); register sets rotate over
    // kPrefetch + 1 strips.
    constexpr int kSets = kPrefetch + 1;
    StripInfo I[kSets];
    Codes C[kSets];
    Scales Sc[kSets];
    if (wave < kProducerWaves) {
        I[0] = run.first;
#pragma unroll
        for (int u = 1; u < kPrefetch; ++u)
            I[u] = (uint32_t)u < n ? next_strip(offs, G, I[u - 1], run.step) : I[u - 1];
#pragma unroll
        for (int u = 0; u < kPrefetch; ++u) {
            Sc[u] = load_scales(scales, K, I[u], kt, soff);
            C[u] = load_codes(codes, K, I[u], kt, coff);
        }
    }

    if (tid < 2 * (kMaxGap + 1))
        lut[tid] = gap_lut_word(tid);
    if (tid == 0) {
        produced = 0;
        published = 0;
        for (int k = 0; k < kSlots; ++k)
            drained[k] = 0;
    }
    __syncthreads();                              // the only barrier: LUT and counters set

    if (wave < kProducerWaves) {
        // ================= producers =================
        // column 32c + j of the tile sits at LDS byte lds_col(32c) + 544 j
        const uint32_t wbase = lds_col(32 * c) + row_q;

        // the lane's four MX scale bytes (zero for rows past the strip: those read as zero)
        struct RowScales {
            uint32_t b[4];
        };
        auto row_scales = [&](const Scales& in) {
            RowScales sc;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                // wave row 4rq + i sits in lanes 2 (4rq + i) and 2 (4rq + i) + 1
                const int src = 2 * (4 * rq + i) + (int)(cl >> 2);
                const uint32_t w = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * src, (int)in.s);
                sc.b[i] = __builtin_amdgcn_ubfe(w, sshift, 8);
            }
            return sc;
        };
        // this wave's max scale of each group over its 32 rows, for the block scale of
        // the strip (combined over the four producer waves once all have published)
        auto publish_max = [&](const RowScales& sc, uint32_t slot) {
            uint32_t m = max(max(sc.b[0], sc.b[1]), max(sc.b[2], sc.b[3]));
            m = max(m, (uint32_t)__builtin_amdgcn_update_dpp((int)m, (int)m, 0x128, 0xF, 0xF, false)); // row_ror:8
            // the 16- and 32-lane swaps of gfx950 (VALU, no LDS round trip)
            const auto a16 = __builtin_amdgcn_permlane16_swap(m, m, false, false);
            m = max((uint32_t)a16[0], (uint32_t)a16[1]);
            const auto a32 = __builtin_amdgcn_permlane32_swap(m, m, false, false);
            m = max((uint32_t)a32[0], (uint32_t)a32[1]);
            if (rq == 0)
                reinterpret_cast<uint8_t*>(pmax[slot])[4 * c + wave] = (uint8_t)m;
        };

        auto produce = [&](const StripInfo& st, const Codes& in, const RowScales& sc, const uint32_t slot,
                           const uint32_t flags) {
            const u8x4 pm = __builtin_bit_cast(u8x4, pmax[slot][c]);
            const uint32_t S = max(max((uint32_t)pm.x, (uint32_t)pm.y), max((uint32_t)pm.z, (uint32_t)pm.w));
            if (wave == 0) {
                if (rq == 0)
                    reinterpret_cast<uint8_t*>(info[slot].S)[c] = (uint8_t)S;
                if (lane == 0) {
                    info[slot].A0 = K * st.row0 + st.r_lo + (int64_t)kTileCols * kt * st.mg;
                    info[slot].mg = (int32_t)st.mg;
                    info[slot].nrows = st.nrows;
                    info[slot].blk = st.s;
                    info[slot].flags = flags;
                }
            }
            // convert each row with its own gap table (even / odd codes apart); rows past
            // the strip have scale 0 and are converted from whatever was loaded: their
            // bytes are never written out
            uint32_t E[4][4], O[4][4];    // [row][code dword]
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t d = min(S - sc.b[i], (uint32_t)kMaxGap);
                const u32x2 t = *reinterpret_cast<const u32x2*>(lut + 2 * d);
                convert8_split(in.c[i].x, t.x, t.y, E[i][0], O[i][0]);
                convert8_split(in.c[i].y, t.x, t.y, E[i][1], O[i][1]);
                convert8_split(in.c[i].z, t.x, t.y, E[i][2], O[i][2]);
                convert8_split(in.c[i].w, t.x, t.y, E[i][3], O[i][3]);
            }
            // code dword q covers columns 8q..8q+7 of the group: even codes -> columns
            // 8q+2mm, odd codes -> 8q+2mm+1; each transposed dword holds the lane's four
            // rows of one column
            uint32_t T[32];               // T[j]: the four rows of column 32c + j
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                transpose4x4(E[0][q], E[1][q], E[2][q], E[3][q], T[8 * q + 0], T[8 * q + 2], T[8 * q + 4], T[8 * q + 6]);
                transpose4x4(O[0][q], O[1][q], O[2][q], O[3][q], T[8 * q + 1], T[8 * q + 3], T[8 * q + 5], T[8 * q + 7]);
            }
            uint8_t* const w = tile + wbase + kStripRows * slot;
#pragma unroll
            for (int j = 0; j < 32; ++j)
                *reinterpret_cast<uint32_t*>(w + kColBytes * j) = T[j];
            // ring bytes 0..31 (rows 0..31 of slot 0) are repeated after the ring, so a
            // 32-byte read window never wraps
            if (slot == 0 && wave == 0) {
#pragma unroll
                for (int j = 0; j < 32; ++j)
                    *reinterpret_cast<uint32_t*>(w + kRing + kColBytes * j) = T[j];
            }
        };
        // a dealt strip neither continues the ring's previous strip nor carries into the next
        auto flags_of = [&](uint32_t prev_sb, const StripInfo& cur, bool lead_in) {
            if (run.dealt)
                return 0u;
            return (prev_sb == cur.sb ? 1u : 0u) | (cur.s + 1 < cur.sb + cur.ns ? 2u : 0u) | (lead_in ? 4u : 0u);
        };

        // Under a full store stream a load takes several strip-times to land.  Step t
        // waits until the consumers have drained strip t - 3 (whose slot carries into
        // strip t - 2, the last reader of slot t % 4) and until all producer waves have
        // published their partial maxima of strip t, converts strip t, signals it, and
        // publishes its own partial maxima of strip t + 1.  The loop is unrolled by the
        // number of register sets so each set keeps fixed registers.
        uint32_t prev_sb = 0xFFFFFFFFu;
        RowScales sc = row_scales(Sc[0]);   // strip t
        publish_max(sc, 0);
        signal(&published);
        for (uint32_t t = 0;; t += kSets) {
#pragma unroll
            for (int u = 0; u < kSets; ++u) {
                const uint32_t tt = t + u;
                const int ld = (u + kPrefetch) % kSets;          // set receiving strip tt + kPrefetch
                const int pv = (u + kPrefetch - 1) % kSets;      // set of strip tt + kPrefetch - 1
                I[ld] = tt + kPrefetch < n ? next_strip(offs, G, I[pv], run.step) : I[pv];
                Sc[ld] = load_scales(scales, K, I[ld], kt, soff);
                C[ld] = load_codes(codes, K, I[ld], kt, coff);
                const int nx = (u + 1) % kSets;                  // set of strip tt + 1
                if (tt >= 3 && !wait_at_least(&drained[(tt - 3) % kSlots],
                                              kConsumerWaves * ((tt - 3) / kSlots + 1), wc))
                    return;
                if (!wait_at_least(&published, kProducerWaves * (tt + 1), wc))
                    return;
                produce(I[u], C[u], sc, tt % kSlots, flags_of(prev_sb, I[u], tt == 0 && run.lead));
                prev_sb = I[u].sb;
                signal(&produced);
                if (tt + 1 >= n)
                    return;
                sc = row_scales(Sc[nx]);
                publish_max(sc, (tt + 1) % kSlots);
                signal(&published);
            }
        }
    }

    // ================= consumers =================
    // the producer waves run in lockstep (each waits for all partial maxima of a strip
    // before converting it), so one summed counter shows that all of them wrote strip t
    consume_strips<kConsumerWaves>(
        tile, info, drained, yT, ncols, n, wave - kProducerWaves,
        [&](uint32_t t) { return wait_at_least(&produced, kProducerWaves * (t + 1), wc); },
        [&](uint32_t slot) {
            if (lane < 16 && 16 * lane < ncols) {
                const uint32_t word = info[slot].S[lane >> 3];
                const uint32_t w4 = ((word >> (8 * ((lane >> 1) & 3))) & 0xFFu) * 0x01010101u;
                *reinterpret_cast<u32x4*>(yT_scales + K * (int64_t)uniform(info[slot].blk) +
                                          kTileCols * (int64_t)kt + 16 * lane) = u32x4{w4, w4, w4, w4};
            }
        });
}

int64_t cols_block_capacity(int64_t M_cap, int32_t G)
{
    return (M_cap + kStripRows - 1) / kStripRows + G;
}

hipError_t launch_fp8_cols(const uint8_t* codes, const uint8_t* scales, uint8_t* yT,
                           uint8_t* yT_scales, const int32_t* offs, int32_t G, int64_t M_cap,
                           int64_t K, WaitCtl wc, hipStream_t stream)
{
    if (M_cap == 0)
        return hipSuccess;
    const int64_t nkt = (K + kTileCols - 1) / kTileCols;
    // one workgroup per compute unit (the LDS ring takes most of a CU's LDS): parts per
    // column tile so that nkt * parts fills the GPU, never more parts than strips
    const int64_t cap_strips = cols_block_capacity(M_cap, G);
    int64_t parts = (int64_t)device_cus() / nkt;
    parts = parts < 1 ? 1 : parts;
    parts = parts > cap_strips ? cap_strips : parts;
    const int64_t grid = nkt * parts;
    if (grid > 0x7FFFFFFF)
        return hipErrorInvalidValue;
    int g = G;
    int64_t k = K;
    int p = (int)parts;
    void* args[] = {(void*)&codes, (void*)&scales, (void*)&yT, (void*)&yT_scales, (void*)&offs,
                    (void*)&g, (void*)&k, (void*)&p, (void*)&wc};
    return launch_kernel((const void*)fp8_cols_kernel, dim3((unsigned)grid), dim3(kColsThreads), args, stream);
}

}  // namespace mxfp4
