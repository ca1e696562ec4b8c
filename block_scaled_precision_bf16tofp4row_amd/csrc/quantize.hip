// quantize.hip -- BF16 -> MXFP4 (E2M1 codes packed two per byte + one UE8M0 scale
// per 32 elements), the row quantizer run right before the expert all-to-all.
//
// Method: "Practical FP4 Training for Large-Scale MoE Models on Hopper GPUs",
// technical summary section 2, item 1 (MXFP4 spec: 32-element blocks, UE8M0 scale,
// E2M1 elements) and item 2 (activations quantized before the all-to-all and packed
// into uint8 containers); the kernel is the page's BF16ToFP4Row (item 3), rebuilt
// for gfx950.  Scale rule and rounding follow OCP MX v1.0 section 6.3: shared
// exponent floor(log2 amax) - 2, E2M1 round-to-nearest-even, saturating at 6; the
// element conversion is gfx950's scaled FP4 convert instruction.
//
// Layout: because K is a multiple of 32, a 32-element block never crosses a row, so
// the [M, K] matrix is a flat stream of blocks: block b reads input bytes
// [64b, 64b+64), writes code bytes [16b, 16b+16) and scale byte b.  One lane takes
// 16 input bytes (8 BF16), a quad of lanes takes one block; the block amax is
// combined across the quad with two DPP steps.  Each lane writes 4 code bytes, so
// a wave's loads (1 KiB) and code stores (256 B) are each one contiguous run.
#include "common.h"

namespace mxfp4 {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Reinterpret a dword as two BF16.  (A __builtin_bit_cast applied directly to an
// ext_vector element such as v.y is lowered as if it named v.x by this compiler, so
// every operand goes through a scalar copy.)
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t u)
{
    bf16x2 r;
    __builtin_memcpy(&r, &u, sizeof(r));
    return r;
}

// Eight BF16 (one 16-byte chunk) -> eight E2M1 codes packed in one dword.
// v_cvt_scalef32_pk_fp4_bf16 converts two BF16 to two E2M1 codes of x / scale with
// round-to-nearest-even and saturation at +-6, keeping the sign (also of zero); the
// low BF16 goes to the low nibble and the byte-select operand picks the destination
// byte, leaving the others as they were.  The scale operand is the fp32 whose
// exponent field is the UE8M0 byte s (only the exponent is used, so s = 0 means
// 2^-127).  This was checked against the oracle for every BF16 pattern and every
// scale byte 0..254.
__device__ __forceinline__ uint32_t encode8(u32x4 v, int s)
{
    const float scale = __uint_as_float((uint32_t)s << 23);
    uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(0u, as_bf16x2(v.x), scale, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(w, as_bf16x2(v.y), scale, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(w, as_bf16x2(v.z), scale, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(w, as_bf16x2(v.w), scale, 3);
    return w;
}

__device__ __forceinline__ uint32_t amax_bits8(u32x4 v)
{
    u16x2 a = __builtin_bit_cast(u16x2, v.x & 0x7FFF7FFFu);
    u16x2 b = __builtin_bit_cast(u16x2, v.y & 0x7FFF7FFFu);
    u16x2 c = __builtin_bit_cast(u16x2, v.z & 0x7FFF7FFFu);
    u16x2 d = __builtin_bit_cast(u16x2, v.w & 0x7FFF7FFFu);
    u16x2 m = __builtin_elementwise_max(__builtin_elementwise_max(a, b), __builtin_elementwise_max(c, d));
    return max((uint32_t)m.x, (uint32_t)m.y);
}

template <int U>
__global__ __launch_bounds__(kThreads) void quantize_rows_kernel(
    const u32x4* __restrict__ x, uint32_t* __restrict__ codes, uint8_t* __restrict__ scales,
    const int32_t* __restrict__ offs, int G, int64_t K)
{
    const int64_t m_tot = offs[G];
    const int64_t nchunks = m_tot * (K / 8);           // 16-byte chunks of 8 BF16
    const int64_t base = (int64_t)blockIdx.x * (kThreads * U);
    if (base >= nchunks)
        return;
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
        // nchunks is a multiple of 4, so a quad is entirely in or out of range and
        // the DPP exchange below never mixes valid and padding lanes of one block.
        uint32_t amax = quad_max_u32(amax_bits8(v[u]));
        int s = max((int)(amax >> 7) - 2, 0);          // biased exponent field - emax(E2M1)
        uint32_t word = encode8(v[u], s);
        if (idx < nchunks) {
            store_stream(codes + idx, word);
            if ((tid & 3) == 0)
                scales[idx >> 2] = (uint8_t)s;
        }
    }
}

// 16-byte chunks per thread (all loads issued before any conversion).  The scale bytes
// stay single-byte stores: gathering a workgroup's 256 of them in LDS for whole 16-byte
// stores (as the row conversion does) needs a barrier at the end, which measured 2-3 %
// slower here.
constexpr int kQuantU = 4;

hipError_t launch_quantize_rows(const uint16_t* x, uint8_t* codes, uint8_t* scales,
                                const int32_t* offs, int32_t G, int64_t M_cap, int64_t K,
                                hipStream_t stream)
{
    int64_t nchunks_cap = M_cap * (K / 8);
    int64_t per_block = (int64_t)kThreads * kQuantU;
    int64_t grid = (nchunks_cap + per_block - 1) / per_block;
    if (grid == 0)
        return hipSuccess;
    if (grid > 0x7FFFFFFF)
        return hipErrorInvalidValue;
    const u32x4* xv = reinterpret_cast<const u32x4*>(x);
    uint32_t* cv = reinterpret_cast<uint32_t*>(codes);
    int g = G;
    int64_t k = K;
    void* args[] = {(void*)&xv, (void*)&cv, (void*)&scales, (void*)&offs, (void*)&g, (void*)&k};
    return launch_kernel((const void*)quantize_rows_kernel<kQuantU>, dim3((unsigned)grid), dim3(kThreads), args,
                         stream);
}

}  // namespace mxfp4
