// fp8q.hip -- the backward FP8 quantizer: BF16 -> FP8 E4M3FN with one UE8M0 scale per
// 1x128 block, row layout (DGRAD operand).
//
// Method: "Practical FP4 Training for Large-Scale MoE Models on Hopper GPUs",
// technical summary section 2: the backward pass of the asymmetric flow (item 2)
// keeps gradients on the standard FP8 path, E4M3 with 128-element blocks (item 1).
// The page does not spell out the block scale; it is read the way the rest of this
// path reads MX scales (OCP MX v1.0 section 6.3 with E4M3's largest exponent 8):
// S = floor(log2 amax) - 8 + 127 clamped to [0, 254], 0 for an all-zero block;
// elements are x / 2^(S-127) rounded to nearest even into the E4M3 subnormals,
// saturating at +-448, sign kept (also of zero).
//
// Layout: K is a multiple of 128, so a 128-block never crosses a row and the [M, K]
// matrix is a flat stream of blocks: block b reads input bytes [256b, 256b+256),
// writes output bytes [128b, 128b+128) and scale byte b.  One lane takes 16 input
// bytes (8 BF16) and writes 8 output bytes; 16 lanes (one DPP row) take one block,
// whose amax is combined with two quad-permute and two row-rotate DPP steps.  A
// wave's loads (1 KiB) and stores (512 B) are each one contiguous run.
//
// Element conversion: v_cvt_scalef32_pk_fp8_bf16 converts two BF16 to two E4M3FN
// bytes of x / scale with round-to-nearest-even (subnormal results included).  It
// does not saturate: a quotient of 464 or more (the midpoint above 448) comes out as
// the NaN byte.  The block maximum divided by 2^(S-127) lies in [256, 512), so
// magnitudes are first clamped to 448 * 2^(S-127), a BF16 number (exponent field
// S + 8 <= 254, mantissa 0x60), which gives the saturated result exactly: quotients
// in (448, 464) round to 448 anyway.  The convert's scale operand is the fp32 2^(S-127)
// (bits S << 23; for S = 0 the subnormal 0x00400000).  This was checked against the
// oracle for every finite BF16 pattern over a spread of scale bytes 0..254.
#include "common.h"

namespace mxfp4 {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short s16x2 __attribute__((ext_vector_type(2)));

namespace {

// DPP row rotations (inside each 16-lane row): row_ror:4 and row_ror:8.
constexpr int kRowRor4 = 0x124;
constexpr int kRowRor8 = 0x128;

__device__ __forceinline__ uint32_t row16_max_u32(uint32_t v)
{
    v = quad_max_u32(v);
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kRowRor4, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kRowRor8, 0xF, 0xF, false));
    return v;
}

__device__ __forceinline__ bf16x2_t bits_as_bf16x2(uint32_t u)
{
    bf16x2_t r;
    __builtin_memcpy(&r, &u, sizeof(r));
    return r;
}

// Largest BF16 magnitude field of eight BF16 (sign bits dropped).
__device__ __forceinline__ uint32_t mag_max8(u32x4 v)
{
    u16x2 a = __builtin_bit_cast(u16x2, v.x & 0x7FFF7FFFu);
    u16x2 b = __builtin_bit_cast(u16x2, v.y & 0x7FFF7FFFu);
    u16x2 c = __builtin_bit_cast(u16x2, v.z & 0x7FFF7FFFu);
    u16x2 d = __builtin_bit_cast(u16x2, v.w & 0x7FFF7FFFu);
    u16x2 m = __builtin_elementwise_max(__builtin_elementwise_max(a, b), __builtin_elementwise_max(c, d));
    return max((uint32_t)m.x, (uint32_t)m.y);
}

// UE8M0 scale byte of a block from the magnitude bits of its amax: the biased
// exponent field minus E4M3's largest exponent (8), at least 0 (a zero or BF16
// subnormal amax, or one below 2^-119, gives 0).
__device__ __forceinline__ int fp8q_scale_of(uint32_t amax_bits)
{
    return max((int)(amax_bits >> 7) - 8, 0);
}

// Two BF16 (one dword) -> two E4M3FN bytes, written into half `hi` of `acc`.  The
// magnitudes are clamped to `clamp2` (the 448 * 2^(S-127) pattern in both halves).
template <bool kHi>
__device__ __forceinline__ s16x2 cvt2(s16x2 acc, uint32_t w, uint32_t clamp2, float scale)
{
    u16x2 mag = __builtin_elementwise_min(__builtin_bit_cast(u16x2, w & 0x7FFF7FFFu),
                                          __builtin_bit_cast(u16x2, clamp2));
    uint32_t c = __builtin_bit_cast(uint32_t, mag) | (w & 0x80008000u);
    return __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(acc, bits_as_bf16x2(c), scale, kHi);
}

// Eight BF16 of one block with scale byte S -> eight E4M3FN bytes in element order.
__device__ __forceinline__ u32x2 fp8q_encode8(u32x4 v, int S)
{
    const uint32_t clamp = ((uint32_t)(S + 8) << 7) | 0x60u;
    const uint32_t clamp2 = clamp | (clamp << 16);
    const float scale = __uint_as_float(S == 0 ? 0x00400000u : (uint32_t)S << 23);
    s16x2 lo = {0, 0}, hi = {0, 0};
    lo = cvt2<false>(lo, v.x, clamp2, scale);
    lo = cvt2<true>(lo, v.y, clamp2, scale);
    hi = cvt2<false>(hi, v.z, clamp2, scale);
    hi = cvt2<true>(hi, v.w, clamp2, scale);
    return u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}

template <int U>
__global__ __launch_bounds__(kThreads) void fp8q_rows_kernel(
    const u32x4* __restrict__ x, u32x2* __restrict__ y, uint8_t* __restrict__ y_scales,
    const int32_t* __restrict__ offs, int G, int64_t K)
{
    // the workgroup's scale bytes (one per 16-lane row), consecutive in y_scales
    constexpr int kScaleBytes = kThreads * U / 16;
    __shared__ __attribute__((aligned(16))) uint8_t sbuf[kScaleBytes];
    const int64_t m_tot = offs[G];
    const int64_t nchunks = m_tot * (K / 8);           // 16-byte chunks of 8 BF16
    const int64_t base = (int64_t)blockIdx.x * (kThreads * U);
    if (base >= nchunks)
        return;                                        // uniform over the workgroup
    const int tid = threadIdx.x;
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        int64_t idx = base + u * kThreads + tid;
        v[u] = idx < nchunks ? load_stream(x + idx) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        int64_t idx = base + u * kThreads + tid;
        // nchunks is a multiple of 16 (K / 8 is), so a 16-lane row is entirely in or
        // out of range and the DPP exchange never mixes valid and padding lanes.
        const int S = fp8q_scale_of(row16_max_u32(mag_max8(v[u])));
        const u32x2 out = fp8q_encode8(v[u], S);
        if (idx < nchunks) {
            store_stream(y + idx, out);
            if ((tid & 15) == 0)
                sbuf[(u * kThreads + tid) >> 4] = (uint8_t)S;
        }
    }
    // The scale bytes go out as whole 16-byte pieces (single-byte stores from every
    // sixteenth lane, spread over workgroups, would each be a partial write to memory).
    // The last workgroup may end inside a piece: its bytes past m_tot * K / 128 stay
    // untouched.
    __syncthreads();
    if (tid < kScaleBytes / 16) {
        const int64_t nb = nchunks >> 4;
        const int64_t p = (base >> 4) + 16 * tid;
        if (p + 16 <= nb)
            store_stream(reinterpret_cast<u32x4*>(y_scales + p), *reinterpret_cast<const u32x4*>(sbuf + 16 * tid));
        else
            for (int q = 0; q < 16 && p + q < nb; ++q)
                y_scales[p + q] = sbuf[16 * tid + q];
    }
}

}  // namespace

// 16-byte chunks per thread (all loads issued before any conversion)
constexpr int kFp8qU = 4;

hipError_t launch_fp8q_rows(const uint16_t* x, uint8_t* y, uint8_t* y_scales,
                            const int32_t* offs, int32_t G, int64_t M_cap, int64_t K,
                            hipStream_t stream)
{
    int64_t nchunks_cap = M_cap * (K / 8);
    int64_t per_block = (int64_t)kThreads * kFp8qU;
    int64_t grid = (nchunks_cap + per_block - 1) / per_block;
    if (grid == 0)
        return hipSuccess;
    if (grid > 0x7FFFFFFF)
        return hipErrorInvalidValue;
    const u32x4* xv = reinterpret_cast<const u32x4*>(x);
    u32x2* yv = reinterpret_cast<u32x2*>(y);
    int g = G;
    int64_t k = K;
    void* args[] = {(void*)&xv, (void*)&yv, (void*)&y_scales, (void*)&offs, (void*)&g, (void*)&k};
    return launch_kernel((const void*)fp8q_rows_kernel<kFp8qU>, dim3((unsigned)grid), dim3(kThreads), args,
                         stream);
}

}  // namespace mxfp4
