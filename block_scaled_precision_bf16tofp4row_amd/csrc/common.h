// common.h -- device helpers shared by the three gfx950 kernels of libmxfp4cvt.
//
// Formats (from "Practical FP4 Training for Large-Scale MoE Models on Hopper GPUs",
// technical summary section 2, item 1): MXFP4 = 32 E2M1 codes (1 sign, 2 exponent,
// 1 mantissa bit) sharing one UE8M0 power-of-two scale; codes are stored two per byte
// (item 2), element 2i in the low nibble.  FP8 target = OCP E4M3FN with one UE8M0
// scale per 128 elements.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxfp4 {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef unsigned char u8x4 __attribute__((ext_vector_type(4)));
// A 16-byte vector with byte alignment: gfx950 global stores accept any byte address.
typedef u32x4 u32x4_unaligned __attribute__((aligned(1)));

constexpr int kThreads = 256;   // 4 wave64 per workgroup

// Bounded waits of the column kernels: the polls a wave makes before it gives up, and
// the device's status word, where a wave that gave up records that it did (the kernels
// only set it; the host reads and clears it).
struct WaitCtl {
    uint32_t* status;
    uint32_t limit;
};
// Polls before a wave gives up by default (about a second of polling): only a broken
// protocol could wait that long.
constexpr uint32_t kDefaultSpinLimit = 1u << 24;

// Every kernel of the library is launched through this (abi.hip).  When the calling
// thread has armed timing events (mxfp4_time_next_launch), the start event is bound to
// the first launch of the next entry-point call and the stop event to the launch with
// last_of_call set (the only one, except in calls that launch two kernels), so their
// elapsed time is the kernels' own execution; then they are disarmed.
hipError_t launch_kernel(const void* kernel, dim3 grid, dim3 block, void** args, hipStream_t stream,
                         bool last_of_call = true);

// ---- memory ---------------------------------------------------------------------

// Every byte of this path is touched exactly once: stream it past the caches.
__device__ __forceinline__ u32x4 load_stream(const u32x4* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ u32x2 load_stream(const u32x2* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void store_stream(u32x4* p, u32x4 v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void store_stream(uint32_t* p, uint32_t v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void store_stream(u32x2* p, u32x2 v) { __builtin_nontemporal_store(v, p); }

// ---- cross-lane -----------------------------------------------------------------

// DPP quad permutations (lanes 4q..4q+3 exchange inside their quad).
constexpr int kQuadSwap1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;  // quad_perm [2,3,0,1]

__device__ __forceinline__ uint32_t quad_max_u32(uint32_t v)
{
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kQuadSwap1, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kQuadSwap2, 0xF, 0xF, false));
    return v;
}

// Byte permute: result byte i = byte sel[i] of the 8-byte value {hi:lo}.
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel)
{
    return __builtin_amdgcn_perm(hi, lo, sel);
}

// ---- E2M1 code -> E4M3FN byte after a scale shift ---------------------------------

// E4M3FN byte of the E2M1 magnitude code c (0..7) multiplied by 2^-d, round to
// nearest even.  Twice the E2M1 magnitude is the integer k below; the value in
// units of 2^-9 (the smallest E4M3 subnormal) is k * 2^(8-d).  Below 16 units the
// E4M3 byte equals the unit count (subnormals and the first normal binade are
// linear in the byte); above, the value is normalised to 8..15 units times 2^(E-1)
// with E the exponent field.  For d > 8 the unit count is k / 2^(d-8), rounded.
constexpr uint8_t e4m3_of_e2m1_shifted(int c, int d)
{
    constexpr int twice[8] = {0, 1, 2, 3, 4, 6, 8, 12};
    int k = twice[c];
    if (k == 0)
        return 0;
    if (d <= 8) {
        int v = k << (8 - d);        // exact: k has at most two significant bits
        int E = 1;
        while (v >= 16) {
            v >>= 1;
            ++E;
        }
        return (uint8_t)(v < 8 ? v : ((E << 3) | (v - 8)));
    }
    int sh = d - 8;
    if (sh >= 8)
        return 0;
    int q = k >> sh;
    int rem = k & ((1 << sh) - 1);
    int half = 1 << (sh - 1);
    if (rem > half || (rem == half && (q & 1)))
        ++q;
    return (uint8_t)q;
}

// Gaps at or above this value flush every code to (signed) zero.
constexpr int kMaxGap = 13;

// The 8-entry byte table for gap d, as two dwords (codes 0..3, codes 4..7).
constexpr uint32_t lut_word(int d, int half)
{
    uint32_t w = 0;
    for (int i = 0; i < 4; ++i)
        w |= (uint32_t)e4m3_of_e2m1_shifted(4 * half + i, d) << (8 * i);
    return w;
}

struct GapLut {
    uint32_t w[kMaxGap + 1][2];
};

constexpr GapLut make_gap_lut()
{
    GapLut t{};
    for (int d = 0; d <= kMaxGap; ++d) {
        t.w[d][0] = lut_word(d, 0);
        t.w[d][1] = lut_word(d, 1);
    }
    return t;
}

// Dword i (0 .. 2 kMaxGap + 1) of the gap table, w[i / 2][i % 2], from immediates: a
// selection over the compile-time table, so staging the table in LDS needs no load from
// memory (a table in constant memory is one more cold round trip before a workgroup's
// first barrier).
__device__ __forceinline__ uint32_t gap_lut_word(int i)
{
    constexpr GapLut t = make_gap_lut();
    uint32_t w = 0;
#pragma unroll
    for (int k = 0; k < 2 * (kMaxGap + 1); ++k)
        w = i == k ? t.w[k >> 1][k & 1] : w;
    return w;
}

// Eight codes (one dword of packed nibbles: byte b holds code 2b in its low nibble and
// code 2b+1 in its high nibble) -> E4M3 bytes, as two dwords: even = codes 0, 2, 4, 6
// and odd = codes 1, 3, 5, 7.  One v_perm_b32 looks up four magnitudes in the 8-byte
// gap table (lut_lo = codes 0..3, lut_hi = codes 4..7); the sign bit of each code
// (bit 3 of its nibble) becomes bit 7 of its byte.
__device__ __forceinline__ void convert8_split(uint32_t w, uint32_t lut_lo, uint32_t lut_hi,
                                               uint32_t& even, uint32_t& odd)
{
    even = perm(lut_hi, lut_lo, w & 0x07070707u) | ((w << 4) & 0x80808080u);
    odd = perm(lut_hi, lut_lo, (w >> 4) & 0x07070707u) | (w & 0x80808080u);
}

// Eight codes -> eight E4M3 bytes in element order (two dwords: codes 0..3, 4..7).
__device__ __forceinline__ u32x2 convert8(uint32_t w, uint32_t lut_lo, uint32_t lut_hi)
{
    uint32_t e, o;
    convert8_split(w, lut_lo, lut_hi, e, o);
    return u32x2{perm(o, e, 0x05010400u), perm(o, e, 0x07030602u)};
}

// ---- workgroup -> XCD-aware tile order ---------------------------------------------

// Workgroups are dispatched round-robin over the 8 XCDs.  Remap so that each XCD
// receives a contiguous range of logical tiles (neighbouring tiles then share an L2).
__device__ __forceinline__ uint32_t xcd_remap(uint32_t bid, uint32_t nblocks)
{
    constexpr uint32_t kXcd = 8;
    uint32_t per = nblocks / kXcd;
    uint32_t full = per * kXcd;
    if (bid >= full)
        return bid;                       // the ragged remainder keeps its order
    return (bid % kXcd) * per + bid / kXcd;
}

}  // namespace mxfp4
