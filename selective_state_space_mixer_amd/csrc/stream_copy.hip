// stream_copy.hip -- a plain device-to-device copy (gfx950): the attainable read+write bandwidth
// that the benchmark reports beside the HBM peak, measured with a kernel of this library's own
// making instead of the runtime's copy.  Each block copies 16 KiB: every thread issues its four
// 16-byte non-temporal loads before its four stores, so each wave keeps 4 KiB in flight.
#include "m2_device.h"
#include "m2_launch.h"

namespace m2 {

constexpr int kCopyThreads = 256;
constexpr int kCopyUnits = 4;  // 16-byte units per thread

__global__ __launch_bounds__(kCopyThreads) void stream_copy_kernel(const u32x4* __restrict__ src,
                                                                   u32x4* __restrict__ dst, int64_t n) {
    const int64_t base = (int64_t)blockIdx.x * (kCopyUnits * kCopyThreads) + threadIdx.x;
    u32x4 v[kCopyUnits];
#pragma unroll
    for (int k = 0; k < kCopyUnits; ++k) {
        const int64_t i = base + k * kCopyThreads;
        if (i < n) v[k] = __builtin_nontemporal_load(src + i);
    }
#pragma unroll
    for (int k = 0; k < kCopyUnits; ++k) {
        const int64_t i = base + k * kCopyThreads;
        if (i < n) __builtin_nontemporal_store(v[k], dst + i);
    }
}

hipError_t launch_stream_copy(void* dst, const void* src, size_t bytes, hipStream_t s) {
    const int64_t n = (int64_t)(bytes / 16);
    if (n == 0) return hipSuccess;
    const int64_t per = (int64_t)kCopyUnits * kCopyThreads;
    const int64_t blocks = (n + per - 1) / per;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    return launch_kernel(stream_copy_kernel, dim3((unsigned)blocks), dim3(kCopyThreads), 0, s,
                         reinterpret_cast<const u32x4*>(src), reinterpret_cast<u32x4*>(dst), n);
}

}  // namespace m2
