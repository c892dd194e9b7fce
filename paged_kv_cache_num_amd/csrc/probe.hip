// Measurement probe: a plain 16-byte-vector device copy of known size, used to
// calibrate HBM byte counters and as the achievable-bandwidth reference.
#include <hip/hip_runtime.h>

#include "kvpool_probe.h"

namespace {

constexpr int kCopyThreads = 256;

__global__ __launch_bounds__(kCopyThreads) void copy_kernel(uint4* __restrict__ dst, const uint4* __restrict__ src,
                                                            uint64_t n) {
    const uint64_t stride = (uint64_t)gridDim.x * kCopyThreads;
    for (uint64_t i = (uint64_t)blockIdx.x * kCopyThreads + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

}  // namespace

extern "C" kv_status kv_probe_copy(void* dst, const void* src, uint64_t bytes, void* stream) {
    if (!dst || !src || (bytes & 15u) || ((reinterpret_cast<uintptr_t>(dst) | reinterpret_cast<uintptr_t>(src)) & 15u))
        return KV_ERR_INVALID_ARGUMENT;
    const uint64_t n = bytes / 16;
    if (n == 0) return KV_OK;
    uint64_t blocks = (n + kCopyThreads - 1) / kCopyThreads;
    if (blocks > 256 * 64) blocks = 256 * 64;   // 64 workgroups per CU, grid-stride for the rest
    copy_kernel<<<dim3((unsigned)blocks), dim3(kCopyThreads), 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<uint4*>(dst), static_cast<const uint4*>(src), n);
    return hipGetLastError() == hipSuccess ? KV_OK : KV_ERR_HIP;
}
