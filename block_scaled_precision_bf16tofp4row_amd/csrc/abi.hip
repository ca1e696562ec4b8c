// abi.hip -- the C ABI of libmxfp4cvt (declared in include/mxfp4cvt.h): synchronous
// argument validation, then the call's kernel launches on the caller's stream (one per
// call, three for the NVFP4 quantizer), all through launch_kernel.
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include <hip/hip_ext.h>

#include "mxfp4cvt.h"
#include "common.h"

namespace mxfp4 {
hipError_t launch_quantize_rows(const uint16_t*, uint8_t*, uint8_t*, const int32_t*, int32_t,
                                int64_t, int64_t, hipStream_t);
hipError_t launch_fp8_rows(const uint8_t*, const uint8_t*, uint8_t*, uint8_t*, const int32_t*,
                           int32_t, int64_t, int64_t, hipStream_t);
hipError_t launch_fp8_cols(const uint8_t*, const uint8_t*, uint8_t*, uint8_t*, const int32_t*,
                           int32_t, int64_t, int64_t, WaitCtl, hipStream_t);
int64_t cols_block_capacity(int64_t M_cap, int32_t G);
hipError_t launch_fp8_gemm(const uint8_t*, const uint8_t*, const uint8_t*, const uint8_t*, uint16_t*,
                           const int32_t*, int32_t, int64_t, int64_t, int64_t, hipStream_t);
hipError_t launch_fp8_wgrad(const uint8_t*, const uint8_t*, const uint8_t*, const uint8_t*, uint16_t*,
                            const int32_t*, int32_t, int64_t, int64_t, int64_t, int64_t, hipStream_t);
hipError_t launch_nvfp4_quantize_rows(const uint16_t*, uint8_t*, uint8_t*, float*, const int32_t*, int32_t,
                                      int64_t, int64_t, bool, uint64_t, hipStream_t);
hipError_t launch_fp8q_cols(const uint16_t*, uint8_t*, uint8_t*, uint8_t*, uint8_t*, const int32_t*, int32_t, int64_t,
                            int64_t, WaitCtl, hipStream_t);
hipError_t launch_fp8q_rows(const uint16_t*, uint8_t*, uint8_t*, const int32_t*, int32_t, int64_t,
                            int64_t, hipStream_t);
}  // namespace mxfp4

namespace {

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Largest M_cap * K the kernels index: every byte count stays far inside int64.
constexpr int64_t kMaxElems = (int64_t)1 << 50;
// Largest K of the column conversion.
constexpr int64_t kMaxColsK = (int64_t)1 << 24;
// Largest N and K of the GEMM (its per-tile byte offsets are 32-bit).
constexpr int64_t kMaxGemmDim = (int64_t)1 << 20;
// Largest width * M_cap of a weight-gradient operand (its byte offsets are 32-bit).
constexpr int64_t kMaxWgradBytes = (int64_t)1 << 30;

mxfp4_status check_shape(int32_t G, int64_t M_cap, int64_t K, int64_t k_multiple)
{
    if (G < 1 || M_cap < 0 || K <= 0 || K % k_multiple != 0)
        return MXFP4_ERR_SHAPE;
    if (M_cap > 0 && K > kMaxElems / M_cap)
        return MXFP4_ERR_SHAPE;
    if (M_cap > INT32_MAX)                   // offsets are int32
        return MXFP4_ERR_SHAPE;
    return MXFP4_OK;
}

mxfp4_status from_hip(hipError_t e) { return e == hipSuccess ? MXFP4_OK : MXFP4_ERR_HIP; }

// ---- bounded-wait give-up status ----------------------------------------------------

// Set (to nonzero) by any column-kernel wave whose bounded wait ran out of polls; each
// device holds its own copy, zero when the code object loads.  Host code uses the
// address hipGetSymbolAddress gives for the device, never this name.
__device__ uint32_t wait_status;

constexpr int kMaxDevices = 64;
std::atomic<uint32_t*> status_addr[kMaxDevices];
std::mutex status_mu;
std::atomic<uint32_t> spin_limit{0};         // 0: the default

// The current device's status word address (looked up once per device).
hipError_t status_word(uint32_t** out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    uint32_t* p = status_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(status_mu);
        p = status_addr[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress((void**)&p, HIP_SYMBOL(wait_status));
            if (e != hipSuccess)
                return e;
            status_addr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return hipSuccess;
}

hipError_t wait_ctl(mxfp4::WaitCtl* w)
{
    const uint32_t lim = spin_limit.load(std::memory_order_relaxed);
    w->limit = lim ? lim : mxfp4::kDefaultSpinLimit;
    return status_word(&w->status);
}

// Copies the current device's status word to *flag, stream-ordered, and waits for it.
hipError_t read_status(uint32_t* flag, hipStream_t stream)
{
    uint32_t* p = nullptr;
    hipError_t e = status_word(&p);
    if (e == hipSuccess)
        e = hipMemcpyAsync(flag, p, sizeof(uint32_t), hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess)
        e = hipStreamSynchronize(stream);
    return e;
}

// Timing events armed by mxfp4_time_next_launch on this thread.
thread_local hipEvent_t armed_start = nullptr;
thread_local hipEvent_t armed_stop = nullptr;

}  // namespace

hipError_t mxfp4::launch_kernel(const void* kernel, dim3 grid, dim3 block, void** args, hipStream_t stream,
                                bool last_of_call)
{
    hipEvent_t start = armed_start;
    hipEvent_t stop = last_of_call ? armed_stop : nullptr;
    if (!start && !stop)
        return hipLaunchKernel(kernel, grid, block, args, 0, stream);
    armed_start = nullptr;
    if (last_of_call)
        armed_stop = nullptr;
    return hipExtLaunchKernel(kernel, grid, block, args, 0, stream, start, stop, 0);
}

extern "C" {

mxfp4_status mxfp4_quantize_rows(const uint16_t* x_bf16, uint8_t* codes, uint8_t* scales,
                                 const int32_t* group_offsets, int32_t G, int64_t M_cap,
                                 int64_t K, hipStream_t stream)
{
    if (!x_bf16 || !codes || !scales || !group_offsets)
        return MXFP4_ERR_NULL;
    mxfp4_status st = check_shape(G, M_cap, K, 32);
    if (st != MXFP4_OK)
        return st;
    if (!aligned(x_bf16, 16) || !aligned(codes, 16) || !aligned(scales, 16) ||
        !aligned(group_offsets, 4))
        return MXFP4_ERR_ALIGN;
    if (M_cap == 0)
        return MXFP4_OK;
    return from_hip(mxfp4::launch_quantize_rows(x_bf16, codes, scales, group_offsets, G, M_cap,
                                                K, stream));
}

static mxfp4_status nvfp4_entry(const uint16_t* x_bf16, uint8_t* codes, uint8_t* scales_e4m3, float* tensor_amax,
                                const int32_t* group_offsets, int32_t G, int64_t M_cap, int64_t K, bool sr,
                                uint64_t seed, hipStream_t stream)
{
    if (!x_bf16 || !codes || !scales_e4m3 || !tensor_amax || !group_offsets)
        return MXFP4_ERR_NULL;
    mxfp4_status st = check_shape(G, M_cap, K, 16);
    if (st != MXFP4_OK)
        return st;
    if (!aligned(x_bf16, 16) || !aligned(codes, 16) || !aligned(scales_e4m3, 16) || !aligned(tensor_amax, 4) ||
        !aligned(group_offsets, 4))
        return MXFP4_ERR_ALIGN;
    return from_hip(mxfp4::launch_nvfp4_quantize_rows(x_bf16, codes, scales_e4m3, tensor_amax, group_offsets, G,
                                                      M_cap, K, sr, seed, stream));
}

mxfp4_status mxfp4_nvfp4_quantize_rows(const uint16_t* x_bf16, uint8_t* codes, uint8_t* scales_e4m3,
                                       float* tensor_amax, const int32_t* group_offsets, int32_t G,
                                       int64_t M_cap, int64_t K, hipStream_t stream)
{
    return nvfp4_entry(x_bf16, codes, scales_e4m3, tensor_amax, group_offsets, G, M_cap, K, false, 0, stream);
}

mxfp4_status mxfp4_nvfp4_quantize_rows_sr(const uint16_t* x_bf16, uint8_t* codes, uint8_t* scales_e4m3,
                                          float* tensor_amax, const int32_t* group_offsets, int32_t G,
                                          int64_t M_cap, int64_t K, uint64_t seed, hipStream_t stream)
{
    return nvfp4_entry(x_bf16, codes, scales_e4m3, tensor_amax, group_offsets, G, M_cap, K, true, seed, stream);
}

mxfp4_status mxfp4_to_fp8_rows(const uint8_t* codes, const uint8_t* scales, uint8_t* y_e4m3,
                               uint8_t* y_scales, const int32_t* group_offsets, int32_t G,
                               int64_t M_cap, int64_t K, hipStream_t stream)
{
    if (!codes || !scales || !y_e4m3 || !y_scales || !group_offsets)
        return MXFP4_ERR_NULL;
    mxfp4_status st = check_shape(G, M_cap, K, 128);
    if (st != MXFP4_OK)
        return st;
    if (!aligned(codes, 16) || !aligned(scales, 16) || !aligned(y_e4m3, 16) ||
        !aligned(y_scales, 16) || !aligned(group_offsets, 4))
        return MXFP4_ERR_ALIGN;
    if (M_cap == 0)
        return MXFP4_OK;
    return from_hip(mxfp4::launch_fp8_rows(codes, scales, y_e4m3, y_scales, group_offsets, G,
                                           M_cap, K, stream));
}

mxfp4_status mxfp4_to_fp8_cols_ragged(const uint8_t* codes, const uint8_t* scales,
                                      uint8_t* yT_e4m3, uint8_t* yT_scales,
                                      const int32_t* group_offsets, int32_t G, int64_t M_cap,
                                      int64_t K, hipStream_t stream)
{
    if (!codes || !scales || !yT_e4m3 || !yT_scales || !group_offsets)
        return MXFP4_ERR_NULL;
    mxfp4_status st = check_shape(G, M_cap, K, 128);
    if (st != MXFP4_OK)
        return st;
    if (K > kMaxColsK)                       // the kernel's per-strip row offsets are 32-bit
        return MXFP4_ERR_SHAPE;
    if (!aligned(codes, 16) || !aligned(scales, 16) || !aligned(yT_e4m3, 16) ||
        !aligned(yT_scales, 16) || !aligned(group_offsets, 4))
        return MXFP4_ERR_ALIGN;
    if (M_cap == 0)
        return MXFP4_OK;
    mxfp4::WaitCtl wc;
    hipError_t e = wait_ctl(&wc);
    if (e == hipSuccess)
        e = mxfp4::launch_fp8_cols(codes, scales, yT_e4m3, yT_scales, group_offsets, G, M_cap, K, wc, stream);
    return from_hip(e);
}

mxfp4_status mxfp4_bf16_to_fp8_rows(const uint16_t* x_bf16, uint8_t* y_e4m3, uint8_t* y_scales,
                                    const int32_t* group_offsets, int32_t G, int64_t M_cap,
                                    int64_t K, hipStream_t stream)
{
    if (!x_bf16 || !y_e4m3 || !y_scales || !group_offsets)
        return MXFP4_ERR_NULL;
    mxfp4_status st = check_shape(G, M_cap, K, 128);
    if (st != MXFP4_OK)
        return st;
    if (!aligned(x_bf16, 16) || !aligned(y_e4m3, 16) || !aligned(y_scales, 16) ||
        !aligned(group_offsets, 4))
        return MXFP4_ERR_ALIGN;
    if (M_cap == 0)
        return MXFP4_OK;
    return from_hip(mxfp4::launch_fp8q_rows(x_bf16, y_e4m3, y_scales, group_offsets, G, M_cap, K,
                                            stream));
}

mxfp4_status mxfp4_bf16_to_fp8_cols_ragged(const uint16_t* x_bf16, uint8_t* yT_e4m3,
                                           uint8_t* yT_scales, const int32_t* group_offsets,
                                           int32_t G, int64_t M_cap, int64_t K,
                                           hipStream_t stream)
{
    if (!x_bf16 || !yT_e4m3 || !yT_scales || !group_offsets)
        return MXFP4_ERR_NULL;
    mxfp4_status st = check_shape(G, M_cap, K, 128);
    if (st != MXFP4_OK)
        return st;
    if (K > kMaxColsK)                       // the kernel's per-strip row offsets are 32-bit
        return MXFP4_ERR_SHAPE;
    if (!aligned(x_bf16, 16) || !aligned(yT_e4m3, 16) || !aligned(yT_scales, 16) ||
        !aligned(group_offsets, 4))
        return MXFP4_ERR_ALIGN;
    if (M_cap == 0)
        return MXFP4_OK;
    mxfp4::WaitCtl wc;
    hipError_t e = wait_ctl(&wc);
    if (e == hipSuccess)
        e = mxfp4::launch_fp8q_cols(x_bf16, yT_e4m3, yT_scales, nullptr, nullptr, group_offsets, G, M_cap, K,
                                    wc, stream);
    return from_hip(e);
}

mxfp4_status mxfp4_bf16_to_fp8_rows_cols_ragged(const uint16_t* x_bf16, uint8_t* y_e4m3, uint8_t* y_scales,
                                                uint8_t* yT_e4m3, uint8_t* yT_scales,
                                                const int32_t* group_offsets, int32_t G, int64_t M_cap,
                                                int64_t K, hipStream_t stream)
{
    if (!x_bf16 || !y_e4m3 || !y_scales || !yT_e4m3 || !yT_scales || !group_offsets)
        return MXFP4_ERR_NULL;
    mxfp4_status st = check_shape(G, M_cap, K, 128);
    if (st != MXFP4_OK)
        return st;
    if (K > kMaxColsK)                       // the kernel's per-strip row offsets are 32-bit
        return MXFP4_ERR_SHAPE;
    if (!aligned(x_bf16, 16) || !aligned(y_e4m3, 16) || !aligned(y_scales, 16) || !aligned(yT_e4m3, 16) ||
        !aligned(yT_scales, 16) || !aligned(group_offsets, 4))
        return MXFP4_ERR_ALIGN;
    if (M_cap == 0)
        return MXFP4_OK;
    mxfp4::WaitCtl wc;
    hipError_t e = wait_ctl(&wc);
    if (e == hipSuccess)
        e = mxfp4::launch_fp8q_cols(x_bf16, yT_e4m3, yT_scales, y_e4m3, y_scales, group_offsets, G, M_cap, K,
                                    wc, stream);
    return from_hip(e);
}

mxfp4_status mxfp4_fp8_grouped_gemm(const uint8_t* a_e4m3, const uint8_t* a_scales,
                                    const uint8_t* w_e4m3, const uint8_t* w_scales,
                                    uint16_t* y_bf16, const int32_t* group_offsets, int32_t G,
                                    int64_t M_cap, int64_t N, int64_t K, hipStream_t stream)
{
    if (!a_e4m3 || !a_scales || !w_e4m3 || !w_scales || !y_bf16 || !group_offsets)
        return MXFP4_ERR_NULL;
    mxfp4_status st = check_shape(G, M_cap, K, 128);
    if (st != MXFP4_OK)
        return st;
    if (K > kMaxGemmDim || N <= 0 || N % 256 != 0 || N > kMaxGemmDim)
        return MXFP4_ERR_SHAPE;
    if (M_cap > 0 && N > kMaxElems / M_cap)          // output elements
        return MXFP4_ERR_SHAPE;
    if ((int64_t)G > kMaxElems / (N * K))             // weight elements
        return MXFP4_ERR_SHAPE;
    if (!aligned(a_e4m3, 16) || !aligned(a_scales, 16) || !aligned(w_e4m3, 16) ||
        !aligned(w_scales, 16) || !aligned(y_bf16, 16) || !aligned(group_offsets, 4))
        return MXFP4_ERR_ALIGN;
    if (M_cap == 0)
        return MXFP4_OK;
    return from_hip(mxfp4::launch_fp8_gemm(a_e4m3, a_scales, w_e4m3, w_scales, y_bf16, group_offsets,
                                           G, M_cap, N, K, stream));
}

mxfp4_status mxfp4_fp8_grouped_gemm_wgrad(const uint8_t* dyT_e4m3, const uint8_t* dyT_scales,
                                          const uint8_t* xT_e4m3, const uint8_t* xT_scales, uint16_t* dw_bf16,
                                          const int32_t* group_offsets, int32_t G, int64_t M_cap, int64_t N,
                                          int64_t K, hipStream_t stream)
{
    if (!dyT_e4m3 || !dyT_scales || !xT_e4m3 || !xT_scales || !dw_bf16 || !group_offsets)
        return MXFP4_ERR_NULL;
    mxfp4_status st = check_shape(G, M_cap, K, 256);
    if (st != MXFP4_OK)
        return st;
    if (N <= 0 || N % 256 != 0 || N > kMaxGemmDim || K > kMaxGemmDim)
        return MXFP4_ERR_SHAPE;
    if (M_cap > 0 && (N > kMaxWgradBytes / M_cap || K > kMaxWgradBytes / M_cap))
        return MXFP4_ERR_SHAPE;
    if ((int64_t)G > kMaxElems / (N * K))             // output elements
        return MXFP4_ERR_SHAPE;
    if (!aligned(dyT_e4m3, 16) || !aligned(dyT_scales, 16) || !aligned(xT_e4m3, 16) ||
        !aligned(xT_scales, 16) || !aligned(dw_bf16, 16) || !aligned(group_offsets, 4))
        return MXFP4_ERR_ALIGN;
    return from_hip(mxfp4::launch_fp8_wgrad(dyT_e4m3, dyT_scales, xT_e4m3, xT_scales, dw_bf16, group_offsets, G,
                                            M_cap, mxfp4::cols_block_capacity(M_cap, G), N, K, stream));
}

int64_t mxfp4_cols_scale_capacity(int64_t M_cap, int64_t K, int32_t G)
{
    if (check_shape(G, M_cap, K, 128) != MXFP4_OK)
        return -1;
    return K * mxfp4::cols_block_capacity(M_cap, G);
}

mxfp4_status mxfp4_validate_offsets(const int32_t* group_offsets, int32_t G, int64_t M_cap,
                                    hipStream_t stream)
{
    if (!group_offsets)
        return MXFP4_ERR_NULL;
    if (G < 1 || M_cap < 0 || M_cap > INT32_MAX)
        return MXFP4_ERR_SHAPE;
    int32_t* h = (int32_t*)malloc(sizeof(int32_t) * ((size_t)G + 1));
    if (!h)
        return MXFP4_ERR_HIP;
    hipError_t e = hipMemcpyAsync(h, group_offsets, sizeof(int32_t) * ((size_t)G + 1),
                                  hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess)
        e = hipStreamSynchronize(stream);
    mxfp4_status st = from_hip(e);
    if (st == MXFP4_OK) {
        if (h[0] != 0)
            st = MXFP4_ERR_SHAPE;
        for (int32_t g = 0; g < G && st == MXFP4_OK; ++g)
            if (h[g + 1] < h[g])
                st = MXFP4_ERR_SHAPE;
        if (st == MXFP4_OK && (int64_t)h[G] > M_cap)
            st = MXFP4_ERR_SHAPE;
    }
    free(h);
    if (st == MXFP4_OK) {
        uint32_t flag = 0;
        st = from_hip(read_status(&flag, stream));
        if (st == MXFP4_OK && flag)
            st = MXFP4_ERR_HIP;
    }
    return st;
}

mxfp4_status mxfp4_wait_status(hipStream_t stream)
{
    uint32_t flag = 0;
    hipError_t e = read_status(&flag, stream);
    if (e == hipSuccess && flag) {
        uint32_t* p = nullptr;
        static const uint32_t zero = 0;
        e = status_word(&p);
        if (e == hipSuccess)
            e = hipMemcpyAsync(p, &zero, sizeof(uint32_t), hipMemcpyHostToDevice, stream);
        if (e == hipSuccess)
            e = hipStreamSynchronize(stream);
    }
    if (e != hipSuccess)
        return MXFP4_ERR_HIP;
    return flag ? MXFP4_ERR_HIP : MXFP4_OK;
}

void mxfp4_set_wait_limit(uint32_t polls) { spin_limit.store(polls, std::memory_order_relaxed); }

mxfp4_status mxfp4_time_next_launch(hipEvent_t start, hipEvent_t stop)
{
    armed_start = start;
    armed_stop = stop;
    return MXFP4_OK;
}

const char* mxfp4_status_string(mxfp4_status status)
{
    switch (status) {
    case MXFP4_OK: return "MXFP4_OK";
    case MXFP4_ERR_NULL: return "MXFP4_ERR_NULL: a required pointer is NULL";
    case MXFP4_ERR_SHAPE: return "MXFP4_ERR_SHAPE: invalid G, M_cap or K";
    case MXFP4_ERR_ALIGN: return "MXFP4_ERR_ALIGN: a pointer is not 16-byte aligned";
    case MXFP4_ERR_HIP: return "MXFP4_ERR_HIP: HIP runtime error";
    }
    return "unknown status";
}

}  // extern "C"
