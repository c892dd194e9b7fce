// Swap of blocks between the pool and pinned host memory.
//
// aicassindra.com "GPU paged KV cache", "Reclaiming memory: swap versus
// recompute" (the victim's blocks are copied to pinned host memory, freed,
// and copied back on resume; the cost is twice the sequence's KV bytes over
// the host link) and "PagedAttention, Internals First", "05 Preemption and
// the scheduler contract" (swap copies the victim's blocks to CPU RAM and
// back).  A sequence's blocks are scattered over the pool, and each (layer,
// tensor) run of a block is only H_kv * B * D * e bytes, so one DMA copy per
// run would pay a command per 4-64 KiB.  Instead one kernel gathers the
// listed blocks and streams them straight into the pinned host buffer through
// its device mapping (16-byte stores over the host link), and one kernel
// streams them back: a single launch per swap, no device staging buffer.
//
// Host buffer layout, per listed block i (stride `block_bytes`, a multiple of
// 16): for each layer l, the K run then the V run (H_kv * B * D * e bytes
// each); then, for FP8 pools, for each layer the K scales then the V scales
// (H_kv fp32 each); zero padding to the stride.  Work items are the 16-byte
// chunks of that layout, so neighbouring lanes move neighbouring bytes on
// both sides.
#include "launch.hpp"

namespace kvp {

namespace {

constexpr int kSwapThreads = 256;

// Where chunk c of block i's host record lives in the pool, or null for padding.
struct SwapMap {
    char* k_base;
    char* v_base;
    uint64_t layer_bytes;
    uint64_t run_bytes;
    const char* k_scale;   // FP8: scale tensors as bytes, else null
    const char* v_scale;
    uint64_t scale_layer_bytes;   // num_blocks * H_kv * 4
    uint64_t scale_run_bytes;     // H_kv * 4
    int32_t num_layers;
};

// Bytes [off, off + 16) of a block record -> pool address (all 16 inside one
// run or one scale run: runs are multiples of 16 bytes, scale runs of 4, and
// the scale section is copied in 4-byte pieces).
__device__ __forceinline__ char* pool_addr(const SwapMap& m, int64_t block, uint64_t off) {
    const uint64_t runs = 2ull * (uint64_t)m.num_layers * m.run_bytes;
    if (off < runs) {
        const uint64_t r = off / m.run_bytes;   // layer * 2 + {K,V}
        const uint64_t in = off - r * m.run_bytes;
        char* base = (r & 1) ? m.v_base : m.k_base;
        return base + (r >> 1) * m.layer_bytes + (uint64_t)block * m.run_bytes + in;
    }
    return nullptr;
}

__device__ __forceinline__ char* scale_addr(const SwapMap& m, int64_t block, uint64_t off) {
    const uint64_t runs = 2ull * (uint64_t)m.num_layers * m.run_bytes;
    const uint64_t s = off - runs;
    if (!m.k_scale || s >= 2ull * (uint64_t)m.num_layers * m.scale_run_bytes) return nullptr;
    const uint64_t r = s / m.scale_run_bytes;
    const uint64_t in = s - r * m.scale_run_bytes;
    const char* base = (r & 1) ? m.v_scale : m.k_scale;
    return const_cast<char*>(base) + (r >> 1) * m.scale_layer_bytes + (uint64_t)block * m.scale_run_bytes + in;
}

template <bool kOut>
__global__ __launch_bounds__(kSwapThreads) void swap_kernel(SwapArgs a, SwapMap m) {
    const int64_t per_block = (int64_t)(a.block_bytes / 16);
    const int64_t total = (int64_t)a.num_list * per_block;
    const int64_t stride = (int64_t)gridDim.x * kSwapThreads;
    const uint64_t runs = 2ull * (uint64_t)m.num_layers * m.run_bytes;
    for (int64_t item = (int64_t)blockIdx.x * kSwapThreads + threadIdx.x; item < total; item += stride) {
        const int64_t i = item / per_block;
        const uint64_t off = (uint64_t)(item - i * per_block) * 16u;
        const int64_t block = a.blocks[i];
        if (block < 0 || block >= a.num_blocks) continue;   // skipped, as in the block copy
        uint4* host = reinterpret_cast<uint4*>(a.host + (uint64_t)i * a.block_bytes + off);
        if (off < runs) {
            uint4* dev = reinterpret_cast<uint4*>(pool_addr(m, block, off));
            if (kOut) *host = *dev;
            else *dev = *host;
        } else {
            // FP8 scales (4-byte runs) and padding: word by word
            uint32_t* hw = reinterpret_cast<uint32_t*>(host);
            uint32_t w[4];
            if (!kOut) {
                const uint4 x = *host;
                w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                uint32_t* d = reinterpret_cast<uint32_t*>(scale_addr(m, block, off + 4u * q));
                if (kOut) w[q] = d ? *d : 0u;
                else if (d) *d = w[q];
            }
            if (kOut) *reinterpret_cast<uint4*>(hw) = make_uint4(w[0], w[1], w[2], w[3]);
        }
    }
}

}  // namespace

hipError_t launch_swap(const SwapArgs& a, bool out, hipStream_t stream) {
    if (a.num_list <= 0) return hipSuccess;
    SwapMap m;
    m.k_base = a.k_base;
    m.v_base = a.v_base;
    m.layer_bytes = a.layer_bytes;
    m.run_bytes = a.run_bytes;
    m.k_scale = reinterpret_cast<const char*>(a.k_scale);
    m.v_scale = reinterpret_cast<const char*>(a.v_scale);
    m.scale_run_bytes = (uint64_t)a.num_kv_heads * 4u;
    m.scale_layer_bytes = (uint64_t)a.num_blocks * m.scale_run_bytes;
    m.num_layers = a.num_layers;
    const int64_t total = (int64_t)a.num_list * (int64_t)(a.block_bytes / 16);
    int64_t blocks = (total + kSwapThreads - 1) / kSwapThreads;
    if (blocks > 8192) blocks = 8192;   // grid-stride over the rest
    if (out) swap_kernel<true><<<dim3((unsigned)blocks), dim3(kSwapThreads), 0, stream>>>(a, m);
    else swap_kernel<false><<<dim3((unsigned)blocks), dim3(kSwapThreads), 0, stream>>>(a, m);
    return hipGetLastError();
}

}  // namespace kvp
