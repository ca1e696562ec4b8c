// nvfp4.hip -- NVFP4 variant quantizer: BF16 -> E2M1 codes in 16-element blocks, one
// E4M3 scale per block under one FP32 scale per tensor.
//
// Format: "Train models faster with JAX and MaxText using NVFP4 on NVIDIA Blackwell",
// the NVFP4 pre-training recipe: 16-element microblocks (half the MXFP4 block), E4M3
// block scales with mantissa bits instead of a power of two, under a per-tensor FP32
// scale; activations and weights round to nearest even.  The arithmetic, in FP32 as the
// recipe's GPU code takes it (the page gives the format, not the formulas):
//   t = FP32(2688 / amax_tensor)    (2688 = 6 * 448; 1 for a zero tensor; FLT_MAX on
//                                    overflow)
//   S = E4M3(FP32(FP32(amax_b / 6) * t)), nearest even, subnormals, saturating at 448
//   e = FP32(t / E4M3value(S))      (0 for S = 0; FLT_MAX on overflow)
//   code = E2M1(FP32(x * e)), nearest even, saturating at 6, sign of x kept.
// The FP32 divisions are IEEE (HIP's default correctly rounded division).
//
// Three launches on the stream: zero the amax word; a grid-stride max of |x| over the
// routed rows (two workgroups per CU), one vector atomic max per workgroup on the float
// bits (non-negative floats order as their bit patterns), skipped when the stored value
// is already as large; the quantizer, which reads the amax, derives t, and
// converts.  The quantizer's layout is the MXFP4 quantizer's with 16-element blocks: a
// lane takes 16 bytes (8 BF16), a lane pair one block, four loads per thread in flight;
// the E4M3 scale is encoded with integer rounding on the FP32 bits (no conversion
// instruction), and the elements with gfx950's scaled FP4 convert at scale 1 (FP32 in,
// nearest even, saturating), after a clamp to [-8, 8] that keeps an overflowed product
// finite without changing its code.
//
// Stochastic rounding (the recipe's gradient quantizers, unbiased): the block scales
// are the same; an element with |y| = |FP32(x * e)| below 6, between the E2M1 values
// lo <= |y| < hi, takes hi when its 16 random bits r satisfy r < 65536 (|y| - lo) /
// (hi - lo), else lo (at or above 6: the code of 6).  The gaps are powers of two, so the
// fraction and the comparison are exact in FP32.  The bits come from Philox4x32-10
// (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC'11)
// keyed by the 64-bit seed, one generator call per 8-element chunk: the counter is the
// chunk's index in the row-major matrix (low word, high word, 0, 0), and element j of
// the chunk takes half j % 2 (0: low) of output word j / 2.  A lane computes its own
// chunk's call, so the conversion is software: the caller picks the mode per call.
#include <float.h>

#include "strips.h"

namespace mxfp4 {

namespace {

constexpr int kNvU = 4;                           // 16-byte chunks per thread in flight
constexpr int kAmaxU = 8;

__device__ __forceinline__ uint32_t nv_max_bits8(u32x4 v)
{
    u16x2 a = __builtin_bit_cast(u16x2, v.x & 0x7FFF7FFFu);
    u16x2 b = __builtin_bit_cast(u16x2, v.y & 0x7FFF7FFFu);
    u16x2 c = __builtin_bit_cast(u16x2, v.z & 0x7FFF7FFFu);
    u16x2 d = __builtin_bit_cast(u16x2, v.w & 0x7FFF7FFFu);
    u16x2 m = __builtin_elementwise_max(__builtin_elementwise_max(a, b), __builtin_elementwise_max(c, d));
    return max((uint32_t)m.x, (uint32_t)m.y);
}

// Non-negative finite v -> E4M3FN magnitude code, nearest even (subnormals included),
// saturating at 0x7E (448).
__device__ __forceinline__ uint32_t e4m3_code_rne_sat(float v)
{
    if (v >= 448.0f)
        return 0x7E;                               // [448, 464] rounds to 448, the rest saturates
    const uint32_t bits = __float_as_uint(v);
    if ((bits >> 23) < 121)                        // below 2^-6: multiples of 2^-9
        return (uint32_t)__builtin_rintf(v * 512.0f);
    const uint32_t r = bits + 0x7FFFFu + ((bits >> 20) & 1u);   // nearest even at 3 mantissa bits
    return (r >> 20) - (120u << 3);                // exponent bias 127 -> 7
}

__device__ __forceinline__ float e4m3_value(uint32_t c)
{
    return c < 8 ? (float)c * (1.0f / 512.0f) : __uint_as_float((((c >> 3) + 120u) << 23) | ((c & 7u) << 20));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

template <int kSel>
__device__ __forceinline__ uint32_t cvt_pair(uint32_t old, float a, float b, float e)
{
    const float ya = __builtin_amdgcn_fmed3f(a * e, -8.0f, 8.0f);
    const float yb = __builtin_amdgcn_fmed3f(b * e, -8.0f, 8.0f);
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, ya, yb, 1.0f, kSel);
}

// Philox4x32-10: ten rounds, each two 32x32 -> 64-bit products of counter words 0 and 2
// with the round constants; the next counter is (hi2 ^ c1 ^ k0, lo2, hi0 ^ c3 ^ k1, lo0)
// and the key advances by the Weyl constants (on the scalar unit: it is wave-uniform).
__device__ __forceinline__ u32x4 philox4x32_10(u32x4 c, uint32_t k0, uint32_t k1)
{
#pragma unroll
    for (int round = 0; round < 10; ++round) {
        const uint64_t p0 = (uint64_t)c.x * 0xD2511F53u;
        const uint64_t p2 = (uint64_t)c.z * 0xCD9E8D57u;
        c = u32x4{(uint32_t)(p2 >> 32) ^ c.y ^ k0, (uint32_t)p2, (uint32_t)(p0 >> 32) ^ c.w ^ k1, (uint32_t)p0};
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return c;
}

// E2M1 code (sign in bit 3) of y rounded stochastically with the random r < 2^16.
// The grid step is 2^(E - 128) with E = max(binade of |y|, 127): 0.5 below 2, 1 in
// [2, 4), 2 from 4.  q = |y| / step is exact (a power-of-two scaling up, or down to at
// least 2); the code is floor(q) + 2 (E - 127), plus one when r < 65536 frac(q) (exact:
// frac(q) is (|y| - lo) / step).  Magnitudes from 6 up reach code 7 or more and are
// clamped; the min with 4 keeps q finite for an overflowed product.
__device__ __forceinline__ uint32_t e2m1_code_sr(float y, uint32_t r)
{
    const uint32_t yb = __float_as_uint(y);
    const uint32_t E = max((yb >> 23) & 0xFFu, 127u);
    const float q = __builtin_fminf(__builtin_ldexpf(__builtin_fabsf(y), 128 - (int)E), 4.0f);
    const float fl = __builtin_floorf(q);
    const uint32_t up = (float)r < (q - fl) * 65536.0f ? 1u : 0u;
    const uint32_t c = min((uint32_t)fl + 2u * (E - 127u) + up, 7u);
    return c | ((yb >> 28) & 8u);
}

}  // namespace

__global__ void nvfp4_amax_init_kernel(uint32_t* __restrict__ amax_bits) { *amax_bits = 0u; }

__global__ __launch_bounds__(kThreads) void nvfp4_amax_kernel(const u32x4* __restrict__ x,
                                                              uint32_t* __restrict__ amax_bits,
                                                              const int32_t* __restrict__ offs, int G, int64_t K)
{
    const int64_t nchunks = (int64_t)offs[G] * (K / 8);
    const int64_t stride = (int64_t)gridDim.x * kThreads * kAmaxU;
    uint32_t m = 0;
    for (int64_t base = (int64_t)blockIdx.x * kThreads * kAmaxU; base < nchunks; base += stride) {
        u32x4 v[kAmaxU];
#pragma unroll
        for (int u = 0; u < kAmaxU; ++u) {
            const int64_t idx = base + u * kThreads + threadIdx.x;
            v[u] = idx < nchunks ? load_stream(x + idx) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < kAmaxU; ++u)
            m = max(m, nv_max_bits8(v[u]));
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1)
        m = max(m, (uint32_t)__shfl_xor((int)m, d, 64));
    // one atomic per workgroup, and none when the stored maximum is already as large:
    // it only grows, so a stale read can cost an atomic but never skip a needed one
    __shared__ uint32_t wave_max[kThreads / 64];
    if ((threadIdx.x & 63) == 0)
        wave_max[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t b = wave_max[0];
#pragma unroll
        for (int w = 1; w < kThreads / 64; ++w)
            b = max(b, wave_max[w]);
        const uint32_t bits = b << 16;             // the BF16 magnitude as FP32 bits
        if (b != 0 && bits > __hip_atomic_load(amax_bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
            atomicMax(amax_bits, bits);
    }
}

template <bool kSR>
__global__ __launch_bounds__(kThreads) void nvfp4_quantize_kernel(const u32x4* __restrict__ x,
                                                                  uint32_t* __restrict__ codes,
                                                                  uint8_t* __restrict__ scales,
                                                                  const uint32_t* __restrict__ amax_bits,
                                                                  const int32_t* __restrict__ offs, int G,
                                                                  int64_t K, uint32_t seed_lo, uint32_t seed_hi)
{
    const int64_t nchunks = (int64_t)offs[G] * (K / 8);
    const int64_t base = (int64_t)blockIdx.x * (kThreads * kNvU);
    if (base >= nchunks)
        return;
    const int tid = threadIdx.x;
    u32x4 v[kNvU];
#pragma unroll
    for (int u = 0; u < kNvU; ++u) {
        const int64_t idx = base + u * kThreads + tid;
        v[u] = idx < nchunks ? load_stream(x + idx) : u32x4{0, 0, 0, 0};
    }
    const float amax = __uint_as_float(*amax_bits);
    float t = amax == 0.0f ? 1.0f : 2688.0f / amax;
    if (!(t <= FLT_MAX))
        t = FLT_MAX;
#pragma unroll
    for (int u = 0; u < kNvU; ++u) {
        const int64_t idx = base + u * kThreads + tid;
        // nchunks is even (K is a multiple of 16), so a lane pair is entirely in or out
        // of range and the exchange below never mixes a valid and a padding lane
        uint32_t mb = nv_max_bits8(v[u]);
        mb = max(mb, (uint32_t)__builtin_amdgcn_mov_dpp((int)mb, 0xB1, 0xF, 0xF, false));  // quad_perm 1,0,3,2
        const float ab = __uint_as_float(mb << 16);
        float sb = ab / 6.0f;
        sb = sb * t;
        const uint32_t S = e4m3_code_rne_sat(sb);
        float e = 0.0f;
        if (S != 0) {
            e = t / e4m3_value(S);
            if (!(e <= FLT_MAX))
                e = FLT_MAX;
        }
        uint32_t w;
        if constexpr (kSR) {
            const u32x4 r = philox4x32_10(u32x4{(uint32_t)idx, (uint32_t)((uint64_t)idx >> 32), 0u, 0u},
                                          seed_lo, seed_hi);
            const uint32_t xs[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
            const uint32_t rs[4] = {r.x, r.y, r.z, r.w};
            w = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                w |= e2m1_code_sr(bf16_lo(xs[q]) * e, rs[q] & 0xFFFFu) << (8 * q);
                w |= e2m1_code_sr(bf16_hi(xs[q]) * e, rs[q] >> 16) << (8 * q + 4);
            }
        } else {
            w = cvt_pair<0>(0u, bf16_lo(v[u].x), bf16_hi(v[u].x), e);
            w = cvt_pair<1>(w, bf16_lo(v[u].y), bf16_hi(v[u].y), e);
            w = cvt_pair<2>(w, bf16_lo(v[u].z), bf16_hi(v[u].z), e);
            w = cvt_pair<3>(w, bf16_lo(v[u].w), bf16_hi(v[u].w), e);
        }
        if (idx < nchunks) {
            store_stream(codes + idx, w);
            if ((tid & 1) == 0)
                scales[idx >> 1] = (uint8_t)S;
        }
    }
}

hipError_t launch_nvfp4_quantize_rows(const uint16_t* x, uint8_t* codes, uint8_t* scales, float* tensor_amax,
                                      const int32_t* offs, int32_t G, int64_t M_cap, int64_t K, bool sr,
                                      uint64_t seed, hipStream_t stream)
{
    const int64_t nchunks_cap = M_cap * (K / 8);
    const u32x4* xv = reinterpret_cast<const u32x4*>(x);
    uint32_t* cv = reinterpret_cast<uint32_t*>(codes);
    uint32_t* ab = reinterpret_cast<uint32_t*>(tensor_amax);
    int g = G;
    int64_t k = K;
    void* iargs[] = {(void*)&ab};
    hipError_t err = launch_kernel((const void*)nvfp4_amax_init_kernel, dim3(1), dim3(1), iargs, stream,
                                   nchunks_cap == 0);
    if (err != hipSuccess || nchunks_cap == 0)
        return err;
    const int64_t per_amax = (int64_t)kThreads * kAmaxU;
    const int64_t grid_amax = min((nchunks_cap + per_amax - 1) / per_amax, (int64_t)(device_cus() * 2));
    void* aargs[] = {(void*)&xv, (void*)&ab, (void*)&offs, (void*)&g, (void*)&k};
    err = launch_kernel((const void*)nvfp4_amax_kernel, dim3((unsigned)grid_amax), dim3(kThreads), aargs, stream,
                        false);
    if (err != hipSuccess)
        return err;
    const int64_t per_block = (int64_t)kThreads * kNvU;
    const int64_t grid = (nchunks_cap + per_block - 1) / per_block;
    if (grid > 0x7FFFFFFF)
        return hipErrorInvalidValue;
    const uint32_t* abc = ab;
    uint32_t seed_lo = (uint32_t)seed, seed_hi = (uint32_t)(seed >> 32);
    void* qargs[] = {(void*)&xv, (void*)&cv,   (void*)&scales,  (void*)&abc,    (void*)&offs,
                     (void*)&g,  (void*)&k, (void*)&seed_lo, (void*)&seed_hi};
    const void* fn = sr ? (const void*)nvfp4_quantize_kernel<true> : (const void*)nvfp4_quantize_kernel<false>;
    return launch_kernel(fn, dim3((unsigned)grid), dim3(kThreads), qargs, stream);
}

}  // namespace mxfp4
