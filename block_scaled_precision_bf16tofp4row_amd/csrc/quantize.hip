// quantize.hip -- BF16 -> MXFP4 (E2M1 codes packed two per byte + one UE8M0 scale
// per 32 elements), the row quantizer run right before the expert all-to-all.
//
// Method: "Practical FP4 Training for Large-Scale MoE Models on Hopper GPUs",
// technical summary section 2, item 1 (MXFP4 spec: 32-element blocks, UE8M0 scale,
// E2M1 elements) and item 2 (activations quantized before the all-to-all and packed
// into uint8 containers); the kernel is the page's BF16ToFP4Row (item 3), rebuilt
// for gfx950.  Scale rule and rounding follow OCP MX v1.0 section 6.3: shared
// exponent floor(log2 amax) - 2, E2M1 round-to-nearest-even, saturating at 6.
//
// Layout: because K is a multiple of 32, a 32-element block never crosses a row, so
// the [M, K] matrix is a flat stream of blocks: block b reads input bytes
// [64b, 64b+64), writes code bytes [16b, 16b+16) and scale byte b.  One lane takes
// 16 input bytes (8 BF16), a quad of lanes takes one block; the block amax is
// combined across the quad with two DPP steps.  Each lane writes 4 code bytes, so
// a wave's loads (1 KiB) and code stores (256 B) are each one contiguous run.
#include "common.h"

namespace mxfp4 {

// E2M1 magnitude code of one BF16 magnitude `mag` (15 bits) in a block with scale
// byte s, i.e. of y = |x| * 2^(127 - s), which lies in [0, 8) because s comes from
// the block amax.  With sig the 8-bit significand (implicit bit included for
// normals) and q = log2 of the E2M1 spacing at y (-1 below 2, 0 in [2, 4), 1 in
// [4, 8)), y / 2^q = sig >> r for r = 7 + q - (exp - s); rounding that to the
// nearest integer n (ties to even) gives code n + 2(q + 1), which saturates at 7.
__device__ __forceinline__ uint32_t e2m1_code(uint32_t mag, int s)
{
    int e = (int)(mag >> 7);
    bool normal = e != 0;
    uint32_t sig = (mag & 0x7Fu) | (normal ? 0x80u : 0u);
    int q = normal ? min(max(e - s - 1, -1), 1) : -1;
    int r = 7 + q - ((normal ? e : 1) - s);
    r = min(r, 9);                           // sig < 256: any shift >= 9 rounds to 0
    uint32_t n = (sig + (1u << (r - 1)) - 1u + ((sig >> r) & 1u)) >> r;
    return min(n + (uint32_t)(2 * (q + 1)), 7u);
}

// Codes of two BF16 in one dword -> one byte (low nibble = low half).
__device__ __forceinline__ uint32_t encode_pair(uint32_t w, int s)
{
    uint32_t lo = w & 0xFFFFu, hi = w >> 16;
    uint32_t c0 = e2m1_code(lo & 0x7FFFu, s) | ((lo >> 12) & 8u);
    uint32_t c1 = e2m1_code(hi & 0x7FFFu, s) | ((hi >> 12) & 8u);
    return c0 | (c1 << 4);
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
        uint32_t word = encode_pair(v[u].x, s) | (encode_pair(v[u].y, s) << 8) |
                        (encode_pair(v[u].z, s) << 16) | (encode_pair(v[u].w, s) << 24);
        if (idx < nchunks) {
            store_stream(codes + idx, word);
            if ((tid & 3) == 0)
                scales[idx >> 2] = (uint8_t)s;
        }
    }
}

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
    return hipLaunchKernel((const void*)quantize_rows_kernel<kQuantU>, dim3((unsigned)grid),
                           dim3(kThreads), args, 0, stream);
}

}  // namespace mxfp4
