// Block copy for copy-on-write.
//
// aicassindra.com "GPU paged KV cache", "Prefix sharing, reference counts,
// and copy-on-write", and "PagedAttention, Internals First", "03 Sharing via
// copy-on-write": a write into a block that more than one table names makes
// the block manager take a fresh block, copy the shared one into it on the
// device, and repoint the writer's table entry; only that one (tail) block is
// ever copied.  This kernel is the device copy: for each (src, dst) pair it
// copies block src to block dst in every layer of the K and the V tensor.
//
// Work items are 16-byte chunks numbered
//     ((pair * layers + layer) * 2 + {K,V}) * block_chunks + chunk,
// a (layer, block) run being H_kv * B * D * e contiguous bytes, so
// neighbouring lanes move neighbouring bytes.  Bit copy, no conversion.  An
// FP8 pool's block scales are copied the same way by a second small kernel.
#include "launch.hpp"

namespace kvp {

namespace {

constexpr int kCopyThreads = 256;

__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(CopyBlocksArgs a) {
    const int64_t per_pair = (int64_t)a.num_layers * 2 * a.block_chunks;
    const int64_t total = (int64_t)a.num_pairs * per_pair;
    const int64_t stride = (int64_t)gridDim.x * kCopyThreads;
    for (int64_t item = (int64_t)blockIdx.x * kCopyThreads + threadIdx.x; item < total; item += stride) {
        const int64_t p = item / per_pair;
        const int64_t rem = item - p * per_pair;
        const int64_t run = rem / a.block_chunks;   // layer * 2 + {K,V}
        const int64_t c = rem - run * a.block_chunks;
        const int layer = (int)(run >> 1);
        const int which = (int)(run & 1);
        const int64_t src = a.pairs[2 * p];
        const int64_t dst = a.pairs[2 * p + 1];
        if (src < 0 || src >= a.num_blocks || dst < 0 || dst >= a.num_blocks) continue;
        uint4* base = reinterpret_cast<uint4*>((which == 0 ? a.k_base : a.v_base) + (uint64_t)layer * a.layer_bytes);
        base[dst * a.block_chunks + c] = base[src * a.block_chunks + c];
    }
}

// FP8 pools: the block scales travel with the block ("PagedAttention,
// Internals First", "06 Open questions": per-block quantization metadata
// rides along with the block, across copy-on-write copies too).  Items
// ((pair * layers + layer) * 2 + {K,V}) * H_kv + head, one fp32 scale each.
__global__ __launch_bounds__(kCopyThreads) void copy_scales_kernel(CopyBlocksArgs a) {
    const int64_t per_pair = (int64_t)a.num_layers * 2 * a.num_kv_heads;
    const int64_t total = (int64_t)a.num_pairs * per_pair;
    const int64_t stride = (int64_t)gridDim.x * kCopyThreads;
    const int64_t layer_elems = (int64_t)a.num_blocks * a.num_kv_heads;
    for (int64_t item = (int64_t)blockIdx.x * kCopyThreads + threadIdx.x; item < total; item += stride) {
        const int64_t p = item / per_pair;
        const int64_t rem = item - p * per_pair;
        const int64_t run = rem / a.num_kv_heads;   // layer * 2 + {K,V}
        const int h = (int)(rem - run * a.num_kv_heads);
        const int64_t src = a.pairs[2 * p];
        const int64_t dst = a.pairs[2 * p + 1];
        if (src < 0 || src >= a.num_blocks || dst < 0 || dst >= a.num_blocks) continue;
        float* base = ((run & 1) == 0 ? a.k_scale : a.v_scale) + (run >> 1) * layer_elems;
        base[dst * a.num_kv_heads + h] = base[src * a.num_kv_heads + h];
    }
}

}  // namespace

hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t stream) {
    if (a.num_pairs <= 0) return hipSuccess;
    const int64_t total = (int64_t)a.num_pairs * a.num_layers * 2 * a.block_chunks;
    int64_t blocks = (total + kCopyThreads - 1) / kCopyThreads;
    if (blocks > 65536) blocks = 65536;   // grid-stride loop covers the rest
    copy_blocks_kernel<<<dim3((unsigned)blocks), dim3(kCopyThreads), 0, stream>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !a.k_scale) return e;
    const int64_t scales = (int64_t)a.num_pairs * a.num_layers * 2 * a.num_kv_heads;
    blocks = (scales + kCopyThreads - 1) / kCopyThreads;
    if (blocks > 65536) blocks = 65536;
    copy_scales_kernel<<<dim3((unsigned)blocks), dim3(kCopyThreads), 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace kvp
