// Launchers shared between the C-ABI layer (kvpool_api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "split.hpp"

namespace kvp {

constexpr int kBlockTokens = 16;   // block size of the fp32 / head_dim-64 decode kernel
constexpr int kTileTokens = 16;    // tokens per K/V tile of the bf16 decode kernels (the MFMA height)
constexpr int kStreamKMaxSeqs = 1024;        // batch size up to which the balanced split is used
constexpr int kStreamKDefaultWorkers = 1024; // worker count when no device can be queried
// Shared-prefix decode: sets of sixteen query columns that one prefix wave
// walks the prefix for (one load of a tile serves all of them).
constexpr int kPrefixSets = 2;
// Column groups of a batch: 16 * kPrefixSets query columns each.
inline int64_t prefix_column_groups(int64_t num_seqs, int64_t group) {
    return ((num_seqs * group + 15) / 16 + kPrefixSets - 1) / kPrefixSets;
}

struct ScatterArgs {
    void* k_layer;               // layer base of the K pool
    void* v_layer;               // layer base of the V pool
    const void* k_new;           // [T][Hkv][D]
    const void* v_new;
    const int64_t* slot_mapping; // [T]
    int64_t num_tokens;
    int64_t num_slots;           // num_blocks * block_size
    int32_t block_size;          // tokens per block (a power of two)
    int32_t block_shift;         // log2(block_size), set by the launcher
    int32_t num_kv_heads;
    int32_t row_chunks;          // 16-byte chunks per (token, head) row = D * elem / 16
    float* k_scale;              // FP8 pools: the layer's scales [num_blocks][Hkv], else null
    float* v_scale;
};

hipError_t launch_scatter(const ScatterArgs& a, hipStream_t stream);
// FP8 pools (head_dim 128, bf16 k_new / v_new): the scales of blocks whose row
// 0 is written, then the quantized rows (fp8_scatter.hip).
hipError_t launch_scatter_fp8(const ScatterArgs& a, hipStream_t stream);

// Decode append: sequence i's new K/V row (k_new[i], v_new[i], [S][Hkv][D]) goes
// to position L_i - 1 of its table, i.e. slot table[i][(L_i - 1) / B] * B +
// (L_i - 1) % B; sequences with L_i = 0 and blocks outside the pool are skipped.
struct AppendArgs {
    void* k_layer;
    void* v_layer;
    const void* k_new;           // [S][Hkv][D]
    const void* v_new;
    const int32_t* tables;       // [S][max_blocks]
    const int32_t* lens;         // [S]
    int32_t max_blocks;
    int32_t num_seqs;
    int32_t num_blocks;
    int32_t max_context;         // clamp for lens[i]
    int32_t num_kv_heads;
    int32_t row_chunks;          // 16-byte chunks per (token, head) row
    int32_t block_size;          // tokens per block
    float* k_scale;              // FP8 pools: the layer's scales [num_blocks][Hkv], else null
    float* v_scale;
};

hipError_t launch_append_scatter(const AppendArgs& a, hipStream_t stream);
hipError_t launch_append_fp8(const AppendArgs& a, hipStream_t stream);

// Copy-on-write block copy: block pairs[2p] -> block pairs[2p + 1] in every
// layer of K and V.  Pairs naming a block outside the pool are skipped.
struct CopyBlocksArgs {
    char* k_base;                // layer 0 of the K tensor
    char* v_base;
    uint64_t layer_bytes;        // bytes per layer of one tensor
    const int32_t* pairs;        // [num_pairs][2] (src, dst)
    int32_t num_pairs;
    int32_t num_layers;
    int32_t num_blocks;
    int64_t block_chunks;        // 16-byte chunks per (layer, block): H_kv * B * D * e / 16
    float* k_scale;              // FP8 pools: layer 0 of the scale tensors [layers][num_blocks][H_kv], else null
    float* v_scale;
    int32_t num_kv_heads;
};

hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t stream);

// Swap: blocks[0..num_list) of every layer (and FP8 scales) to / from a host
// buffer the device can address, block_bytes per listed block.
struct SwapArgs {
    char* k_base;                // layer 0 of the K tensor
    char* v_base;
    uint64_t layer_bytes;
    uint64_t run_bytes;          // one (layer, block) run of one tensor: H_kv * B * D * e
    float* k_scale;              // FP8: layer 0 of the scale tensors, else null
    float* v_scale;
    const int32_t* blocks;       // device, [num_list]
    char* host;                  // device address of the host buffer
    uint64_t block_bytes;        // host record per listed block (multiple of 16)
    int32_t num_list;
    int32_t num_layers;
    int32_t num_blocks;
    int32_t num_kv_heads;
};

hipError_t launch_swap(const SwapArgs& a, bool out, hipStream_t stream);

struct DecodeArgs {
    SplitConsts split;           // balanced split and partitions on its workers: W, weights, reciprocals
    const void* k_layer;
    const void* v_layer;
    const void* q;               // [S][Hq][D]
    void* out;                   // [S][Hq][D]
    const int32_t* tables;       // [S][max_blocks]
    const int32_t* lens;         // [S]
    float* ws_ml;                // partitions: [S][Hq][max_parts] x (m, l), or null
    float* ws_acc;               // partitions: [S][Hq][max_parts][D]; balanced split: partial records
    int64_t* ws_prefix;          // balanced split: tiles before each sequence, [S + 1]
    const void* k_append;        // balanced split, decode append: new row per sequence [S][Hkv][D], or null
    const void* v_append;
    const float* k_scale;        // FP8 pools: the layer's block scales [num_blocks][Hkv]
    const float* v_scale;
    // balanced split: other rows stored by extra waves of the same launch
    // (reshape_and_cache semantics, FP8 pools with the block scale rule; slots
    // the attention does not read)
    const void* rows_k;          // [num_rows][Hkv][D]
    const void* rows_v;
    const int64_t* rows_slots;   // [num_rows]
    int64_t num_rows;
    int32_t append_waves;        // balanced split: extra waves storing the decode rows (set by the launcher)
    int32_t workers;             // balanced split: worker waves (the launch adds append / row waves past them)
    int32_t piece_cost;          // balanced split: positions before each (sequence, KV head) walk's tiles
    int32_t max_blocks;
    int32_t num_seqs;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t num_blocks;
    int32_t block_size;          // tokens per block: 16 for every kernel; 8..128 for the bf16 ones
    int32_t max_context;         // clamp for lens[i]
    int32_t part_tokens;         // tokens per partition (multiple of 16)
    int32_t max_parts;           // ceil(max_context / part_tokens), >= 1
    float scale_log2;            // softmax scale * log2(e)
    // Shared prefix (paged_attention_decode_shared, bf16, block sizes 8..128): the
    // first shared_tiles table entries of every sequence name the same blocks.
    // The prefix waves leave (m, l, output) per (sequence, query head) and
    // part in slots 0 .. prefix_parts-1 of ws_pml / ws_pacc ([S][Hq][parts + 1]
    // x (m, l) and x head_dim); the balanced kernel walks only the tiles past
    // the prefix and leaves a (sequence, KV head) it covers whole in slot
    // prefix_parts; the fix-up merges them.  shared_tiles 0: none of this.
    int32_t shared_tiles;
    int32_t shared_entries;      // table entries those tiles take: shared_tiles * 16 / block_size
    int32_t prefix_parts;
    int32_t prefix_part_tiles;   // tiles per part (the last part may have fewer)
    float* ws_pml;
    float* ws_pacc;
};

// dtype: 0 fp32, 1 bf16, 2 FP8 E4M3.  Returns hipErrorInvalidValue for a shape without a kernel.
hipError_t launch_decode(const DecodeArgs& a, int dtype, int head_dim, hipStream_t stream);
bool decode_shape_supported(int dtype, int head_dim, int group, int block_size);

// bf16 pools with head_dim 128: scores on the matrix cores (decode_mfma.hip).
// Launches the decode kernel only; the caller launches the partition merge.
hipError_t launch_decode_bf16_mfma(const DecodeArgs& a, int group, hipStream_t stream);
// The same kernels reading an FP8 pool (codes widened to bf16, block scales
// applied to the scores and the probabilities); block sizes 8..128.
hipError_t launch_decode_fp8_mfma(const DecodeArgs& a, int group, hipStream_t stream);

// bf16 / head_dim 128, balanced split over `workers` single-wave workers plus
// the fix-up of split (sequence, KV head) pairs; no partition merge needed.
hipError_t launch_decode_bf16_streamk(const DecodeArgs& a, int group, int workers, hipStream_t stream);
// The same with a shared prefix (a.shared_tiles > 0): prefix waves beside the
// balanced decode of what follows the prefix, then the fix-up merging both.
hipError_t launch_decode_bf16_shared(const DecodeArgs& a, int group, int workers, hipStream_t stream);
hipError_t launch_decode_fp8_streamk(const DecodeArgs& a, int group, int workers, hipStream_t stream);
// head_dim 128, at most kStreamKMaxSeqs sequences, partition_size > 0: the
// (sequence, KV head, partition) items on the balanced split's workers, one
// wave per item; the caller launches the partition merge.
hipError_t launch_decode_bf16_partitions(const DecodeArgs& a, int group, int workers, hipStream_t stream);
hipError_t launch_decode_fp8_partitions(const DecodeArgs& a, int group, int workers, hipStream_t stream);
// the partition merge for bf16 outputs (decode.hip)
hipError_t launch_partition_merge_bf16(const DecodeArgs& a, hipStream_t stream);
// Worker count for the balanced split on the current device (resident waves:
// one per SIMD for bf16 tiles, two for FP8 tiles).
int streamk_workers(int group, bool fp8);

}  // namespace kvp
