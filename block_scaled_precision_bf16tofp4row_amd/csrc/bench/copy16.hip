// copy16.hip -- libmxfp4bench: a plain streaming device copy in 16-byte pieces, the
// memory-system ceiling the benchmark sets beside each conversion kernel (a kernel
// that reads R bytes and writes W bytes is compared with this copy moving the same
// R + W bytes).  Not part of libmxfp4cvt.
//
// One-shot grid: thread t of workgroup b moves pieces b * 256 U + u * 256 + t for
// u < U, all loads issued before the stores, both streaming past the caches (each byte
// is touched once), the same access shape as the row kernels.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

template <int U>
__global__ __launch_bounds__(kThreads) void copy16_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                          int64_t n)
{
    const int64_t base = (int64_t)blockIdx.x * (kThreads * U) + threadIdx.x;
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t i = base + (int64_t)u * kThreads;
        v[u] = i < n ? __builtin_nontemporal_load(src + i) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t i = base + (int64_t)u * kThreads;
        if (i < n)
            __builtin_nontemporal_store(v[u], dst + i);
    }
}

template <int U>
hipError_t launch(const void* src, void* dst, int64_t n, hipStream_t stream, hipEvent_t start, hipEvent_t stop)
{
    const int64_t per = (int64_t)kThreads * U;
    const int64_t grid = (n + per - 1) / per;
    if (grid == 0)
        return hipSuccess;
    if (grid > 0x7FFFFFFF)
        return hipErrorInvalidValue;
    const u32x4* s = static_cast<const u32x4*>(src);
    u32x4* d = static_cast<u32x4*>(dst);
    void* args[] = {(void*)&s, (void*)&d, (void*)&n};
    if (start || stop)
        return hipExtLaunchKernel((const void*)copy16_kernel<U>, dim3((unsigned)grid), dim3(kThreads), args, 0,
                                  stream, start, stop, 0);
    return hipLaunchKernel((const void*)copy16_kernel<U>, dim3((unsigned)grid), dim3(kThreads), args, 0, stream);
}

}  // namespace

// Copies n16 16-byte pieces from src to dst (device pointers, 16-byte aligned, not
// overlapping) on `stream`, each thread moving `unroll` pieces (1, 2, 4 or 8).  `start`
// and `stop` (either may be NULL) are bound to the kernel's own start and end
// (hipExtLaunchKernel), as the conversion library's timing hook binds them to its
// kernels.  Returns 0 when the launch was enqueued, -1 for bad arguments, else the HIP
// error.
extern "C" int bench_copy16(void* dst, const void* src, int64_t n16, int unroll, hipStream_t stream,
                            hipEvent_t start, hipEvent_t stop)
{
    if (!dst || !src || n16 <= 0 || ((uintptr_t)dst & 15) || ((uintptr_t)src & 15))
        return -1;
    hipError_t e;
    switch (unroll) {
    case 1: e = launch<1>(src, dst, n16, stream, start, stop); break;
    case 2: e = launch<2>(src, dst, n16, stream, start, stop); break;
    case 4: e = launch<4>(src, dst, n16, stream, start, stop); break;
    case 8: e = launch<8>(src, dst, n16, stream, start, stop); break;
    default: return -1;
    }
    return (int)e;
}

// Timing events for the benchmark: created with timing enabled, owned by the caller.
extern "C" hipEvent_t bench_event_create(void)
{
    hipEvent_t e = nullptr;
    return hipEventCreate(&e) == hipSuccess ? e : nullptr;
}

extern "C" void bench_event_destroy(hipEvent_t e)
{
    if (e)
        (void)hipEventDestroy(e);
}

// Waits for `stop` and returns the time from `start` to `stop` in microseconds, or a
// negative value when either event has not completed a recording.
extern "C" double bench_event_elapsed_us(hipEvent_t start, hipEvent_t stop)
{
    float ms = 0.0f;
    if (hipEventSynchronize(stop) != hipSuccess || hipEventElapsedTime(&ms, start, stop) != hipSuccess)
        return -1.0;
    return 1000.0 * (double)ms;
}
