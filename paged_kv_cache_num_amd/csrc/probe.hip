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

constexpr int kReadBlocks = 256 * 32;   // 32 workgroups per compute unit, grid-stride

__global__ __launch_bounds__(kCopyThreads) void read_kernel(const uint4* __restrict__ src, uint64_t n,
                                                            uint32_t* __restrict__ sink) {
    const uint64_t stride = (uint64_t)gridDim.x * kCopyThreads;
    uint32_t acc = 0;
    for (uint64_t i = (uint64_t)blockIdx.x * kCopyThreads + threadIdx.x; i < n; i += stride) {
        const uint4 x = src[i];
        acc ^= x.x ^ x.y ^ x.z ^ x.w;
    }
    // fold the wave, then one word per workgroup
    for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
    __shared__ uint32_t part[kCopyThreads / 64];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t v = 0;
        for (int w = 0; w < kCopyThreads / 64; ++w) v ^= part[w];
        sink[blockIdx.x % (65536 / 4)] = v;
    }
}

}  // namespace

extern "C" kv_status kv_probe_read(const void* src, uint64_t bytes, void* sink, void* stream) {
    if (!src || !sink || (bytes & 15u) || (reinterpret_cast<uintptr_t>(src) & 15u) || (reinterpret_cast<uintptr_t>(sink) & 3u))
        return KV_ERR_INVALID_ARGUMENT;
    const uint64_t n = bytes / 16;
    if (n == 0) return KV_OK;
    uint64_t blocks = (n + kCopyThreads - 1) / kCopyThreads;
    if (blocks > kReadBlocks) blocks = kReadBlocks;
    read_kernel<<<dim3((unsigned)blocks), dim3(kCopyThreads), 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<const uint4*>(src), n, static_cast<uint32_t*>(sink));
    return hipGetLastError() == hipSuccess ? KV_OK : KV_ERR_HIP;
}

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
