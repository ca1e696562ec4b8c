// cols_traffic.hip -- libmxfp4bench: the memory traffic of a transposed-column kernel
// with nothing else, the ceiling the benchmark sets beside the column kernels.
//
// The column kernels read 128-row strips of a 256-column tile (128 code bytes, or 512
// BF16 bytes, of each row, plus the strip's MX scale bytes for the FP4 input)
// and write, for each of the tile's columns, the 128-byte output line the strip covers
// in the expert's transposed layout, plus the tile's 256 block-scale bytes of the strip.
// This kernel issues exactly those loads and stores as a one-shot grid, one workgroup
// per (tile, strip), with no conversion, no LDS and no synchronisation.  Workgroups go
// tile by tile over consecutive strips (the order in which the running workgroups write
// neighbouring lines of the same columns, the fastest order measured for this traffic),
// and every store writes a whole aligned line (the line holding the strip's first byte
// of the column).  The stored values depend on every loaded value, so no load is dead.
// With `sequential` set, the same loads are followed by stores of the same size to one
// contiguous 32 KB block per workgroup: what the reads cost next to untransposed writes.
// Not part of libmxfp4cvt.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kTileCols = 256;
constexpr int kStripRows = 128;

// P: 16-byte input pieces per thread (4 for 128 input bytes per tile row, 16 for 512).
template <int P>
__global__ __launch_bounds__(kThreads) void cols_traffic_kernel(
    const uint8_t* __restrict__ in, int64_t in_pitch, const uint8_t* __restrict__ sc, int64_t sc_pitch,
    uint8_t* __restrict__ out, int64_t out_bytes, uint8_t* __restrict__ out_scales,
    const int64_t* __restrict__ strips, uint32_t nstrips, int64_t K, int sequential)
{
    constexpr int kRowPieces = P * kThreads / kStripRows;     // 16-byte pieces per tile row
    const uint32_t kt = blockIdx.x / nstrips;
    const uint32_t s = blockIdx.x % nstrips;
    const int64_t row = strips[4 * s + 0];
    const int64_t nrows = strips[4 * s + 1];
    const int64_t A0 = strips[4 * s + 2];
    const int64_t mg = strips[4 * s + 3];
    const int ncols = (int)min<int64_t>(kTileCols, K - (int64_t)kTileCols * kt);
    const int row_pieces = kRowPieces * ncols / kTileCols;    // narrow last tile: half the row
    const int tid = threadIdx.x;

    u32x4 v[P];
#pragma unroll
    for (int u = 0; u < P; ++u) {
        const int i = u * kThreads + tid;
        const int r = i / kRowPieces, c = i % kRowPieces;
        v[u] = u32x4{0, 0, 0, 0};
        if (r < nrows && c < row_pieces)
            v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
                in + (row + r) * in_pitch + (int64_t)kt * (kRowPieces * 16) + 16 * c));
    }
    u32x4 acc = v[0];
#pragma unroll
    for (int u = 1; u < P; ++u)
        acc ^= v[u];
    // The MX scale bytes of the strip's rows (one contiguous block, sc_pitch a multiple of
    // 4) are read once, as whole dwords, by the workgroups of tile 0: reading each tile's
    // 8 bytes per row in this tile-by-tile order would fetch every row's scale sector once
    // per tile, far more than the column kernel's traffic (its workgroups on the same
    // strips of all tiles run at the same time).
    if (sc && kt == 0) {
        const uint32_t* p = reinterpret_cast<const uint32_t*>(sc + row * sc_pitch);
        const int64_t n4 = nrows * sc_pitch / 4;
        for (int64_t i = tid; i < n4; i += kThreads)
            acc.x ^= __builtin_nontemporal_load(p + i);
    }

    // 8 lanes per column line, 8 columns per store instruction
#pragma unroll
    for (int u = 0; u < kTileCols * 8 / kThreads; ++u) {
        const int j = u * kThreads + tid;
        const int k = j >> 3, c = j & 7;
        if (k >= ncols)
            continue;
        int64_t at;
        if (sequential) {
            at = ((int64_t)blockIdx.x * kTileCols + k) * 128 + 16 * c;
        } else {
            const int64_t A = A0 + ((int64_t)kTileCols * kt + k) * mg;
            at = (A & ~(int64_t)127) + 16 * c;
        }
        if (at + 16 > out_bytes)
            continue;
        u32x4 w = acc;
        w.x ^= (uint32_t)j;
        __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(out + at));
    }
    if (tid < kTileCols / 16 && 16 * tid < ncols) {
        u32x4 w = acc;
        w.y ^= (uint32_t)tid;
        __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(out_scales + (int64_t)s * K +
                                                                  (int64_t)kTileCols * kt + 16 * tid));
    }
}

}  // namespace

// Moves the traffic of a transposed-column kernel over `nstrips` strips (see the top of
// this file).  in: rows of `in_pitch` bytes, of which a 256-column tile reads
// `tile_in_bytes` (128: MXFP4 codes, or 512: BF16) per row; sc: the MX scale rows
// (`sc_pitch` bytes) or NULL; out: `out_bytes` bytes, stores past them are dropped;
// out_scales: nstrips * K bytes.  strips: device int64 [nstrips][4] = first input row,
// rows (1..128), output byte of (column 0, the strip's first row), and the expert's row
// count (the column stride).  K a multiple of 128 with 128-byte-aligned rows.  `start`
// and `stop` (either may be NULL) are bound to the kernel's start and end.  Returns 0
// when the launch was enqueued, -1 for bad arguments, else the HIP error.
extern "C" int bench_cols_traffic(const void* in, int64_t in_pitch, int tile_in_bytes, const void* sc,
                                  int64_t sc_pitch, void* out, int64_t out_bytes, void* out_scales,
                                  const int64_t* strips, int64_t nstrips, int64_t K, int sequential,
                                  hipStream_t stream, hipEvent_t start, hipEvent_t stop)
{
    if (!in || !out || !out_scales || !strips || nstrips <= 0 || nstrips > 0x7FFFFFFF || K <= 0 || K % 128 ||
        (tile_in_bytes != 128 && tile_in_bytes != 512) || in_pitch != K * tile_in_bytes / kTileCols ||
        (sc && sc_pitch != K / 32) || ((uintptr_t)in & 15) || ((uintptr_t)out & 15) ||
        ((uintptr_t)out_scales & 15))
        return -1;
    const int64_t nkt = (K + kTileCols - 1) / kTileCols;
    const int64_t grid = nkt * nstrips;
    if (grid > 0x7FFFFFFF)
        return -1;
    const uint8_t* a = static_cast<const uint8_t*>(in);
    const uint8_t* b = static_cast<const uint8_t*>(sc);
    uint8_t* o = static_cast<uint8_t*>(out);
    uint8_t* os = static_cast<uint8_t*>(out_scales);
    uint32_t ns = (uint32_t)nstrips;
    int seq = sequential ? 1 : 0;
    void* args[] = {(void*)&a, (void*)&in_pitch, (void*)&b, (void*)&sc_pitch, (void*)&o, (void*)&out_bytes,
                    (void*)&os, (void*)&strips, (void*)&ns, (void*)&K, (void*)&seq};
    const void* kern = tile_in_bytes == 128 ? (const void*)cols_traffic_kernel<4> : (const void*)cols_traffic_kernel<16>;
    if (start || stop)
        return (int)hipExtLaunchKernel(kern, dim3((unsigned)grid), dim3(kThreads), args, 0, stream, start, stop, 0);
    return (int)hipLaunchKernel(kern, dim3((unsigned)grid), dim3(kThreads), args, 0, stream);
}
