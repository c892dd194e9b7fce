// C ABI of the paged KV-cache hot path: argument checks, launch set-up, errors.
// The operations themselves are described in include/kvpool.h.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>

#include "kvpool.h"
#include "host_logic.hpp"
#include "launch.hpp"
#include "split.hpp"

struct kv_pool {
    kv_pool_desc desc;
    char* k_base;
    char* v_base;
    uint64_t layer_bytes;   // bytes of one layer of one tensor
    int32_t elem_bytes;
    float* k_scale;         // FP8 pools: [layers][blocks][kv_heads] fp32, else null
    float* v_scale;
    uint64_t scale_layer;   // scale entries per layer (blocks * kv_heads)
};

namespace {

thread_local char g_last_error[512] = "";

kv_status fail(kv_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return s;
}

kv_status ok() {
    g_last_error[0] = '\0';
    return KV_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_bytes_of(int32_t dtype) { return kvp::host::elem_bytes_of(dtype); }

// a host_logic.hpp status, its message recorded as the last error
kv_status from_host(kv_status s, const kvp::host::Message& m) { return s == KV_OK ? ok() : fail(s, "%s", m.text); }

#if defined(KV_DEBUG) && KV_DEBUG
constexpr bool kDebugChecks = true;    // host-side precondition checks of the debug build
#else
constexpr bool kDebugChecks = false;
#endif

kv_status hip_fail(hipError_t e, const char* what) {
    return fail(KV_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

uint64_t round_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

// How one decode call is laid out; shared by the workspace query and the launch.
enum class Mode { kSingle, kPartitions, kBalanced };

struct Plan {
    Mode mode;
    int32_t part_tokens;   // tokens per partition (kSingle: covers max_context_len)
    int32_t max_parts;
    int32_t workers;       // kBalanced only
    uint64_t ws_first;     // bytes of the first workspace region (ml pairs, or tile prefix sums)
    uint64_t ws_total;
};

Plan plan_decode(const kv_pool_desc& d, int32_t num_seqs, int32_t num_q_heads, int32_t max_context_len,
                 int32_t partition_size) {
    Plan p;
    memset(&p, 0, sizeof p);
    const int group = num_q_heads / d.num_kv_heads;
    // the balanced split counts its positions in 32 bits: at most
    // ceil(max_context_len / 16) tiles plus the walk-start positions per
    // (sequence, KV head)
    const int64_t max_cost = kvp::kBf16PieceCost > kvp::kFp8PieceCost ? kvp::kBf16PieceCost : kvp::kFp8PieceCost;
    const int64_t positions = (int64_t)num_seqs * d.num_kv_heads *
                              (((int64_t)max_context_len + kvp::kTileTokens - 1) / kvp::kTileTokens + max_cost);
    if (partition_size == 0 && (d.dtype == KV_BF16 || d.dtype == KV_FP8_E4M3) && d.head_dim == 128 &&
        num_seqs <= kvp::kStreamKMaxSeqs && positions < kvp::kMaxSplitPositions) {
        p.mode = Mode::kBalanced;
        p.workers = kvp::streamk_workers(group, d.dtype == KV_FP8_E4M3);
        p.part_tokens = 0;
        p.max_parts = 1;
        p.ws_first = round_up((uint64_t)(num_seqs + 1) * 8u, 256u);
        // two partial records per worker: group x head_dim outputs, then (m, l) per head padded to 16 bytes
        const uint64_t rec_floats = (uint64_t)group * (uint64_t)d.head_dim + (uint64_t)((2 * group + 3) / 4) * 4u;
        p.ws_total = p.ws_first + 2ull * (uint64_t)p.workers * rec_floats * 4u;
        return p;
    }
    if (partition_size == 0 || partition_size >= max_context_len) {
        const uint64_t unit = d.block_size > kvp::kTileTokens ? (uint64_t)d.block_size : (uint64_t)kvp::kTileTokens;
        int32_t whole = (int32_t)round_up((uint64_t)(max_context_len > 0 ? max_context_len : 1), unit);
        p.mode = Mode::kSingle;
        p.part_tokens = partition_size > whole ? partition_size : whole;
        p.max_parts = 1;
        return p;
    }
    p.mode = Mode::kPartitions;
    p.part_tokens = partition_size;
    p.max_parts = (max_context_len + partition_size - 1) / partition_size;
    // bf16 / FP8 pools with head_dim 128: the partitions run on the balanced split's workers
    if ((d.dtype == KV_BF16 || d.dtype == KV_FP8_E4M3) && d.head_dim == 128 && num_seqs <= kvp::kStreamKMaxSeqs)
        p.workers = kvp::streamk_workers(group, d.dtype == KV_FP8_E4M3);
    // (m, l) pairs first, then the fp32 partial outputs at a 256-byte boundary
    const uint64_t entries = (uint64_t)num_seqs * (uint64_t)num_q_heads * (uint64_t)p.max_parts;
    p.ws_first = round_up(entries * 8u, 256u);
    p.ws_total = p.ws_first + entries * (uint64_t)d.head_dim * 4u;
    return p;
}

// A shared-prefix call: the balanced plan, then the prefix states
// [S][Hq][parts + 1] x (m, l) and x head_dim.  The prefix is cut into parts
// so that about one prefix wave runs for every two workers of the balanced
// split (they share the launch), every part non-empty.  On the 128-sequence
// prefix-sharing batch (4 parts of 32 tiles, 512 prefix waves) the call took
// 44.8 us on one layer back to back, against 57.5 / 49.8 / 47.0 / 49.6 us
// with 2 / 3 / 6 / 8 parts.
struct SharedPlan {
    Plan base;
    int32_t parts;
    int32_t part_tiles;
    uint64_t pml_off, pacc_off, total;
};

// 16-token tiles the prefix waves take for a prefix of shared_blocks blocks:
// whole tiles only (with 8-token blocks an odd last block goes to the
// per-sequence walks, which read it like any other block).
int32_t shared_tiles_of(const kv_pool_desc& d, int32_t shared_blocks) {
    return (int32_t)((int64_t)shared_blocks * d.block_size / kvp::kTileTokens);
}

SharedPlan plan_shared(const kv_pool_desc& d, int32_t num_seqs, int32_t num_q_heads, int32_t max_context_len,
                       int32_t shared_tiles) {
    SharedPlan sp;
    memset(&sp, 0, sizeof sp);
    sp.base = plan_decode(d, num_seqs, num_q_heads, max_context_len, 0);
    const int64_t group = num_q_heads / d.num_kv_heads;
    const int64_t column_groups = kvp::prefix_column_groups(num_seqs, group) * d.num_kv_heads;
    const int64_t want = ((int64_t)sp.base.workers / 2 + column_groups - 1) / (column_groups > 0 ? column_groups : 1);
    int64_t parts = want < 1 ? 1 : (want > shared_tiles ? shared_tiles : want);
    sp.part_tiles = (int32_t)((shared_tiles + parts - 1) / parts);
    sp.parts = (int32_t)((shared_tiles + sp.part_tiles - 1) / sp.part_tiles);
    const uint64_t states = (uint64_t)num_seqs * (uint64_t)num_q_heads * (uint64_t)(sp.parts + 1);
    sp.pml_off = round_up(sp.base.ws_total, 256u);
    sp.pacc_off = sp.pml_off + round_up(states * 8u, 256u);
    sp.total = sp.pacc_off + states * (uint64_t)d.head_dim * 4u;
    return sp;
}

// Shapes the shared-prefix kernels cover.
kv_status check_shared(const kv_pool_desc& d, int32_t num_seqs, int32_t max_context_len, int32_t max_blocks_per_seq,
                       int32_t shared_blocks) {
    if (shared_blocks < 0) return fail(KV_ERR_INVALID_ARGUMENT, "shared_blocks %d < 0", shared_blocks);
    if (shared_blocks == 0) return KV_OK;
    if (d.dtype != KV_BF16 || d.head_dim != 128)
        return fail(KV_ERR_UNSUPPORTED, "a shared prefix needs a bf16 pool with head_dim 128");
    if (num_seqs > kvp::kStreamKMaxSeqs)
        return fail(KV_ERR_UNSUPPORTED, "a shared prefix is handled for at most %d sequences", kvp::kStreamKMaxSeqs);
    if (plan_decode(d, num_seqs, d.num_kv_heads, max_context_len, 0).mode != Mode::kBalanced)
        return fail(KV_ERR_UNSUPPORTED, "a shared prefix needs the balanced split, which counts at most %lld positions",
                    (long long)kvp::kMaxSplitPositions);
    if (shared_blocks > max_blocks_per_seq || (int64_t)shared_blocks * d.block_size > max_context_len)
        return fail(KV_ERR_INVALID_ARGUMENT, "shared_blocks %d exceeds max_blocks_per_seq %d or max_context_len %d / %d",
                    shared_blocks, max_blocks_per_seq, max_context_len, d.block_size);
    return KV_OK;
}

// Arguments of a batch of rows to store (reshape_and_cache and the rows of
// paged_attention_decode_step).
kv_status check_rows(kv_pool_t pool, const void* k_new, const void* v_new, const int64_t* slot_mapping,
                     int64_t num_tokens) {
    if (num_tokens < 0) return fail(KV_ERR_INVALID_ARGUMENT, "num_tokens %lld < 0", (long long)num_tokens);
    if (num_tokens == 0) return ok();
    if (!k_new || !v_new || !slot_mapping) return fail(KV_ERR_INVALID_ARGUMENT, "NULL device pointer");
    if (!aligned16(k_new) || !aligned16(v_new)) return fail(KV_ERR_INVALID_ARGUMENT, "k_new/v_new must be 16-byte aligned");
    if (reinterpret_cast<uintptr_t>(slot_mapping) & 7u) return fail(KV_ERR_INVALID_ARGUMENT, "slot_mapping must be 8-byte aligned");
    if (pool->desc.num_kv_heads > (1 << 20))   // the kernels number a token's chunks in 32 bits
        return fail(KV_ERR_UNSUPPORTED, "num_kv_heads %d above 2^20", pool->desc.num_kv_heads);
    return ok();
}

// The scatter kernel for num_tokens > 0 checked rows (FP8 pools: quantized, with block scales).
hipError_t launch_rows(kv_pool_t pool, int32_t layer, const void* k_new, const void* v_new,
                       const int64_t* slot_mapping, int64_t num_tokens, void* stream) {
    kvp::ScatterArgs a;
    memset(&a, 0, sizeof a);
    a.k_layer = pool->k_base + (uint64_t)layer * pool->layer_bytes;
    a.v_layer = pool->v_base + (uint64_t)layer * pool->layer_bytes;
    a.k_new = k_new;
    a.v_new = v_new;
    a.slot_mapping = slot_mapping;
    a.num_tokens = num_tokens;
    a.num_slots = (int64_t)pool->desc.num_blocks * pool->desc.block_size;
    a.block_size = pool->desc.block_size;
    a.num_kv_heads = pool->desc.num_kv_heads;
    a.row_chunks = pool->desc.head_dim * pool->elem_bytes / 16;
    if (pool->desc.dtype == KV_FP8_E4M3) {
        a.k_scale = pool->k_scale + (uint64_t)layer * pool->scale_layer;
        a.v_scale = pool->v_scale + (uint64_t)layer * pool->scale_layer;
        return kvp::launch_scatter_fp8(a, static_cast<hipStream_t>(stream));
    }
    return kvp::launch_scatter(a, static_cast<hipStream_t>(stream));
}

}  // namespace

extern "C" {

const char* kv_status_string(kv_status status) {
    switch (status) {
        case KV_OK: return "KV_OK";
        case KV_ERR_INVALID_ARGUMENT: return "KV_ERR_INVALID_ARGUMENT";
        case KV_ERR_UNSUPPORTED: return "KV_ERR_UNSUPPORTED";
        case KV_ERR_WORKSPACE_TOO_SMALL: return "KV_ERR_WORKSPACE_TOO_SMALL";
        case KV_ERR_HIP: return "KV_ERR_HIP";
        case KV_ERR_OUT_OF_RANGE: return "KV_ERR_OUT_OF_RANGE";
    }
    return "KV_ERR_UNKNOWN";
}

const char* kv_last_error_message(void) { return g_last_error; }

kv_status kv_pool_bytes(const kv_pool_desc* desc, uint64_t* bytes_per_tensor) {
    if (!bytes_per_tensor) return fail(KV_ERR_INVALID_ARGUMENT, "bytes_per_tensor is NULL");
    kvp::host::Message m;
    return from_host(kvp::host::pool_bytes(desc, bytes_per_tensor, m), m);
}

kv_status kv_pool_scale_bytes(const kv_pool_desc* desc, uint64_t* bytes_per_tensor) {
    if (!bytes_per_tensor) return fail(KV_ERR_INVALID_ARGUMENT, "bytes_per_tensor is NULL");
    kvp::host::Message m;
    return from_host(kvp::host::scale_bytes(desc, bytes_per_tensor, m), m);
}

namespace {

kv_status create_pool(const kv_pool_desc* desc, void* k_base, void* v_base, float* k_scales, float* v_scales,
                      kv_pool_t* out) {
    if (!out) return fail(KV_ERR_INVALID_ARGUMENT, "out is NULL");
    *out = nullptr;
    uint64_t total = 0;
    kv_status s = kv_pool_bytes(desc, &total);
    if (s != KV_OK) return s;
    if (!k_base || !v_base) return fail(KV_ERR_INVALID_ARGUMENT, "pool base pointer is NULL");
    if (!aligned16(k_base) || !aligned16(v_base)) return fail(KV_ERR_INVALID_ARGUMENT, "pool base pointers must be 16-byte aligned");
    const bool fp8 = desc->dtype == KV_FP8_E4M3;
    if (fp8 && (!k_scales || !v_scales ||
                ((reinterpret_cast<uintptr_t>(k_scales) | reinterpret_cast<uintptr_t>(v_scales)) & 3u)))
        return fail(KV_ERR_INVALID_ARGUMENT, "FP8 scale tensors must be non-NULL and 4-byte aligned");
    const int32_t B = desc->block_size;
    if (B != 8 && B != 16 && B != 32 && B != 64 && B != 128)
        return fail(KV_ERR_UNSUPPORTED, "block_size %d: kernels are built for 8, 16, 32, 64 and 128", B);
    if (B != kvp::kBlockTokens && !((desc->dtype == KV_BF16 || fp8) && desc->head_dim == 128))
        return fail(KV_ERR_UNSUPPORTED, "block_size %d needs a bf16 or FP8 pool with head_dim 128 (other pools use %d)",
                    B, kvp::kBlockTokens);
    if (desc->head_dim != 64 && desc->head_dim != 128)
        return fail(KV_ERR_UNSUPPORTED, "head_dim %d: kernels are built for 64 and 128", desc->head_dim);
    if (fp8 && desc->head_dim != 128) return fail(KV_ERR_UNSUPPORTED, "FP8 pools are built for head_dim 128");
    kv_pool* p = new (std::nothrow) kv_pool;
    if (!p) return fail(KV_ERR_INVALID_ARGUMENT, "out of host memory");
    p->desc = *desc;
    p->k_base = static_cast<char*>(k_base);
    p->v_base = static_cast<char*>(v_base);
    p->layer_bytes = total / (uint64_t)desc->num_layers;
    p->elem_bytes = elem_bytes_of(desc->dtype);
    p->k_scale = fp8 ? k_scales : nullptr;
    p->v_scale = fp8 ? v_scales : nullptr;
    p->scale_layer = (uint64_t)desc->num_blocks * (uint64_t)desc->num_kv_heads;
    *out = p;
    return ok();
}

}  // namespace

kv_status kv_pool_create(const kv_pool_desc* desc, void* k_base, void* v_base, kv_pool_t* out) {
    if (desc && desc->dtype == KV_FP8_E4M3) {
        if (out) *out = nullptr;
        return fail(KV_ERR_INVALID_ARGUMENT, "FP8 pools carry scale tensors: create them with kv_pool_create_fp8");
    }
    return create_pool(desc, k_base, v_base, nullptr, nullptr, out);
}

kv_status kv_pool_create_fp8(const kv_pool_desc* desc, void* k_codes, void* v_codes, float* k_scales,
                             float* v_scales, kv_pool_t* out) {
    if (desc && desc->dtype != KV_FP8_E4M3) {
        if (out) *out = nullptr;
        return fail(KV_ERR_INVALID_ARGUMENT, "kv_pool_create_fp8 needs dtype KV_FP8_E4M3");
    }
    return create_pool(desc, k_codes, v_codes, k_scales, v_scales, out);
}

kv_status kv_pool_destroy(kv_pool_t pool) {
    delete pool;
    return ok();
}

kv_status kv_build_slot_mapping(const int32_t* block_tables, int32_t num_rows, int32_t max_blocks_per_seq,
                                int32_t block_size, int32_t num_blocks, const int32_t* write_seq,
                                const int32_t* write_start, const int32_t* write_count, int32_t num_requests,
                                int64_t* slot_mapping, int64_t capacity, int64_t* num_tokens) {
    kvp::host::Message m;
    return from_host(kvp::host::build_slot_mapping(block_tables, num_rows, max_blocks_per_seq, block_size, num_blocks,
                                                   write_seq, write_start, write_count, num_requests, slot_mapping,
                                                   capacity, num_tokens, kDebugChecks, m),
                     m);
}

kv_status reshape_and_cache(kv_pool_t pool, int32_t layer, const void* k_new, const void* v_new,
                            const int64_t* slot_mapping, int64_t num_tokens, void* stream) {
    if (!pool) return fail(KV_ERR_INVALID_ARGUMENT, "pool is NULL");
    if (layer < 0 || layer >= pool->desc.num_layers)
        return fail(KV_ERR_INVALID_ARGUMENT, "layer %d outside [0, %d)", layer, pool->desc.num_layers);
    const kv_status st = check_rows(pool, k_new, v_new, slot_mapping, num_tokens);
    if (st != KV_OK || num_tokens == 0) return st;
    const hipError_t e = launch_rows(pool, layer, k_new, v_new, slot_mapping, num_tokens, stream);
    if (e != hipSuccess) return hip_fail(e, "scatter launch");
    return ok();
}

kv_status kv_copy_blocks(kv_pool_t pool, const int32_t* block_pairs, int32_t num_pairs, void* stream) {
    if (!pool) return fail(KV_ERR_INVALID_ARGUMENT, "pool is NULL");
    if (num_pairs < 0) return fail(KV_ERR_INVALID_ARGUMENT, "num_pairs %d < 0", num_pairs);
    if (num_pairs == 0) return ok();
    if (!block_pairs) return fail(KV_ERR_INVALID_ARGUMENT, "block_pairs is NULL");
    if (reinterpret_cast<uintptr_t>(block_pairs) & 3u) return fail(KV_ERR_INVALID_ARGUMENT, "block_pairs must be 4-byte aligned");
    const kv_pool_desc& d = pool->desc;
    kvp::CopyBlocksArgs a;
    memset(&a, 0, sizeof a);
    a.k_base = pool->k_base;
    a.v_base = pool->v_base;
    a.layer_bytes = pool->layer_bytes;
    a.pairs = block_pairs;
    a.num_pairs = num_pairs;
    a.num_layers = d.num_layers;
    a.num_blocks = d.num_blocks;
    a.block_chunks = (int64_t)d.num_kv_heads * d.block_size * d.head_dim * pool->elem_bytes / 16;
    a.k_scale = pool->k_scale;   // null unless FP8
    a.v_scale = pool->v_scale;
    a.num_kv_heads = d.num_kv_heads;
    hipError_t e = kvp::launch_copy_blocks(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "copy_blocks launch");
    return ok();
}

}  // extern "C"

namespace {

// Host record of one swapped block: the 2 * layers runs, then FP8 scales, padded to 16 bytes.
uint64_t swap_record_bytes(const kv_pool* p) {
    const kv_pool_desc& d = p->desc;
    const uint64_t run = (uint64_t)d.num_kv_heads * d.block_size * d.head_dim * p->elem_bytes;
    uint64_t rec = 2ull * d.num_layers * run;
    if (p->k_scale) rec += 2ull * d.num_layers * d.num_kv_heads * 4u;
    return round_up(rec, 16u);
}

kv_status swap_impl(kv_pool_t pool, const int32_t* blocks, int32_t num_blocks, const void* host, uint64_t host_bytes,
                    bool out, void* stream) {
    const char* what = out ? "kv_swap_out" : "kv_swap_in";
    if (!pool) return fail(KV_ERR_INVALID_ARGUMENT, "%s: pool is NULL", what);
    if (num_blocks < 0) return fail(KV_ERR_INVALID_ARGUMENT, "%s: num_blocks %d < 0", what, num_blocks);
    if (num_blocks == 0) return ok();
    if (!blocks || (reinterpret_cast<uintptr_t>(blocks) & 3u))
        return fail(KV_ERR_INVALID_ARGUMENT, "%s: blocks must be a non-NULL, 4-byte aligned device pointer", what);
    if (!host || !aligned16(host)) return fail(KV_ERR_INVALID_ARGUMENT, "%s: host buffer must be non-NULL and 16-byte aligned", what);
    const uint64_t rec = swap_record_bytes(pool);
    if (host_bytes < rec * (uint64_t)num_blocks)
        return fail(KV_ERR_INVALID_ARGUMENT, "%s: host buffer of %llu bytes, %llu needed", what,
                    (unsigned long long)host_bytes, (unsigned long long)(rec * (uint64_t)num_blocks));
    // the kernels address the host buffer through its device mapping: it must be pinned host memory
    hipPointerAttribute_t attr;
    memset(&attr, 0, sizeof attr);
    hipError_t e = hipPointerGetAttributes(&attr, host);
    if (e != hipSuccess || attr.type != hipMemoryTypeHost) {
        (void)hipGetLastError();
        return fail(KV_ERR_INVALID_ARGUMENT, "%s: the host buffer is not pinned host memory (hipHostMalloc)", what);
    }
    void* mapped = nullptr;
    e = hipHostGetDevicePointer(&mapped, const_cast<void*>(host), 0);
    if (e != hipSuccess || !mapped) {
        (void)hipGetLastError();
        return fail(KV_ERR_INVALID_ARGUMENT, "%s: the host buffer has no device mapping", what);
    }
    const kv_pool_desc& d = pool->desc;
    kvp::SwapArgs a;
    memset(&a, 0, sizeof a);
    a.k_base = pool->k_base;
    a.v_base = pool->v_base;
    a.layer_bytes = pool->layer_bytes;
    a.run_bytes = (uint64_t)d.num_kv_heads * d.block_size * d.head_dim * pool->elem_bytes;
    a.k_scale = pool->k_scale;
    a.v_scale = pool->v_scale;
    a.blocks = blocks;
    a.host = static_cast<char*>(mapped);
    a.block_bytes = rec;
    a.num_list = num_blocks;
    a.num_layers = d.num_layers;
    a.num_blocks = d.num_blocks;
    a.num_kv_heads = d.num_kv_heads;
    e = kvp::launch_swap(a, out, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, what);
    return ok();
}

}  // namespace

extern "C" {

kv_status kv_swap_bytes(kv_pool_t pool, int32_t num_blocks, uint64_t* bytes) {
    if (!pool || !bytes) return fail(KV_ERR_INVALID_ARGUMENT, "NULL argument");
    *bytes = 0;
    if (num_blocks < 0) return fail(KV_ERR_INVALID_ARGUMENT, "num_blocks %d < 0", num_blocks);
    *bytes = swap_record_bytes(pool) * (uint64_t)num_blocks;
    return ok();
}

kv_status kv_swap_out(kv_pool_t pool, const int32_t* blocks, int32_t num_blocks, void* host, uint64_t host_bytes,
                      void* stream) {
    return swap_impl(pool, blocks, num_blocks, host, host_bytes, true, stream);
}

kv_status kv_swap_in(kv_pool_t pool, const int32_t* blocks, int32_t num_blocks, const void* host, uint64_t host_bytes,
                     void* stream) {
    return swap_impl(pool, blocks, num_blocks, host, host_bytes, false, stream);
}

kv_status paged_attention_workspace_bytes(kv_pool_t pool, int32_t num_seqs, int32_t num_q_heads,
                                          int32_t max_context_len, int32_t partition_size, uint64_t* bytes) {
    if (!pool || !bytes) return fail(KV_ERR_INVALID_ARGUMENT, "NULL argument");
    *bytes = 0;
    if (num_seqs < 0 || num_q_heads <= 0 || max_context_len < 0 || partition_size < 0)
        return fail(KV_ERR_INVALID_ARGUMENT, "negative size argument");
    const int32_t unit = pool->desc.block_size > kvp::kTileTokens ? pool->desc.block_size : kvp::kTileTokens;
    if (partition_size % unit != 0)
        return fail(KV_ERR_INVALID_ARGUMENT, "partition_size %d is not a multiple of %d (the block size and the 16-token tile)",
                    partition_size, unit);
    if (num_q_heads % pool->desc.num_kv_heads != 0)
        return fail(KV_ERR_INVALID_ARGUMENT, "num_q_heads %d is not a multiple of num_kv_heads %d", num_q_heads,
                    pool->desc.num_kv_heads);
    *bytes = plan_decode(pool->desc, num_seqs, num_q_heads, max_context_len, partition_size).ws_total;
    return ok();
}

}  // extern "C"

namespace {

// Workspace of paged_attention_decode_noalloc: one static array per device.
// In host code `scratch` only names the symbol; its device address on each
// GPU comes from hipGetSymbolAddress, looked up once per device and kept.
constexpr uint64_t kScratchBytes = KV_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kScratchMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kScratchMaxDevices];

// Device address of `scratch` on device `dev`, looked up with that device
// current (the caller's current device is restored).
kv_status scratch_on_device(int dev, void** ptr) {
    if (dev < 0 || dev >= kScratchMaxDevices)
        return fail(KV_ERR_HIP, "device %d: the static workspace is kept for devices 0..%d", dev, kScratchMaxDevices - 1);
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p) {
        *ptr = p;
        return KV_OK;
    }
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return hip_fail(e, "hipSetDevice");
    const hipError_t look = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev && (e = hipSetDevice(cur)) != hipSuccess) return hip_fail(e, "hipSetDevice (restore)");
    if (look != hipSuccess || !p) return hip_fail(look != hipSuccess ? look : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
    // several host threads may look it up at once: they find the same address
    g_scratch_ptr[dev].store(p, std::memory_order_release);
    *ptr = p;
    return KV_OK;
}

// Device of `stream` (the current device for the null stream).
kv_status stream_device(void* stream, int* dev) {
    hipError_t e;
    if (stream) {
        hipDevice_t d = 0;
        e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &d);
        *dev = (int)d;
    } else {
        e = hipGetDevice(dev);
    }
    return e == hipSuccess ? KV_OK : hip_fail(e, "device of the stream");
}

// Shared body of paged_attention_decode, paged_attention_decode_append,
// paged_attention_decode_shared and paged_attention_decode_noalloc (k_append
// / v_append null but for the append call; static_scratch: the workspace is
// the stream's device's static array, once every argument has been checked).
kv_status decode_impl(kv_pool_t pool, int32_t layer, void* out, const void* q, const void* k_append,
                      const void* v_append, const int32_t* block_tables, int32_t max_blocks_per_seq,
                      const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads, float scale,
                      int32_t max_context_len, int32_t partition_size, void* workspace, uint64_t workspace_bytes,
                      void* stream, int32_t shared_blocks = 0, bool static_scratch = false,
                      const void* rows_k = nullptr, const void* rows_v = nullptr, const int64_t* rows_slots = nullptr,
                      int64_t num_rows = 0) {
    if (!pool) return fail(KV_ERR_INVALID_ARGUMENT, "pool is NULL");
    const kv_pool_desc& d = pool->desc;
    if (layer < 0 || layer >= d.num_layers) return fail(KV_ERR_INVALID_ARGUMENT, "layer %d outside [0, %d)", layer, d.num_layers);
    {
        const kv_status st = check_rows(pool, rows_k, rows_v, rows_slots, num_rows);
        if (st != KV_OK) return st;
    }
    if (num_seqs < 0 || max_context_len < 0 || partition_size < 0 || max_blocks_per_seq <= 0)
        return fail(KV_ERR_INVALID_ARGUMENT, "negative size argument");
    if (num_q_heads <= 0 || num_q_heads % d.num_kv_heads != 0)
        return fail(KV_ERR_INVALID_ARGUMENT, "num_q_heads %d is not a positive multiple of num_kv_heads %d", num_q_heads,
                    d.num_kv_heads);
    const int group = num_q_heads / d.num_kv_heads;
    if (!kvp::decode_shape_supported(d.dtype, d.head_dim, group, d.block_size))
        return fail(KV_ERR_UNSUPPORTED, "query group size %d: kernels are built for 1, 2, 4 and 8", group);
    const int32_t unit = d.block_size > kvp::kTileTokens ? d.block_size : kvp::kTileTokens;
    if (partition_size % unit != 0)
        return fail(KV_ERR_INVALID_ARGUMENT, "partition_size %d is not a multiple of %d (the block size and the 16-token tile)",
                    partition_size, unit);
    if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * d.block_size)
        return fail(KV_ERR_INVALID_ARGUMENT, "max_context_len %d exceeds max_blocks_per_seq * block_size = %lld",
                    max_context_len, (long long)max_blocks_per_seq * d.block_size);
    if (!std::isfinite(scale) || !(scale > 0.0f)) return fail(KV_ERR_INVALID_ARGUMENT, "scale must be finite and positive");
    if (num_seqs > 65535 || num_q_heads > 65535)
        return fail(KV_ERR_UNSUPPORTED, "num_seqs %d / num_q_heads %d above the 65535 grid limit", num_seqs, num_q_heads);
    if (num_seqs == 0) {   // nothing to attend; other rows are still stored
        if (num_rows == 0) return ok();
        const hipError_t e = launch_rows(pool, layer, rows_k, rows_v, rows_slots, num_rows, stream);
        return e == hipSuccess ? ok() : hip_fail(e, "scatter launch");
    }
    if (!out || !q || !block_tables || !context_lens) return fail(KV_ERR_INVALID_ARGUMENT, "NULL device pointer");
    if (!aligned16(out) || !aligned16(q)) return fail(KV_ERR_INVALID_ARGUMENT, "q/out must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(block_tables) | reinterpret_cast<uintptr_t>(context_lens)) & 3u)
        return fail(KV_ERR_INVALID_ARGUMENT, "block_tables/context_lens must be 4-byte aligned");
    const bool append = k_append != nullptr || v_append != nullptr;
    if (append && (!k_append || !v_append || !aligned16(k_append) || !aligned16(v_append)))
        return fail(KV_ERR_INVALID_ARGUMENT, "k_new/v_new must both be non-NULL and 16-byte aligned");

    if (shared_blocks > 0) {
        const kv_status st = check_shared(d, num_seqs, max_context_len, max_blocks_per_seq, shared_blocks);
        if (st != KV_OK) return st;
    }
    const int32_t stiles = shared_blocks > 0 ? shared_tiles_of(d, shared_blocks) : 0;   // 0: the plain call
    const SharedPlan sp = stiles > 0 ? plan_shared(d, num_seqs, num_q_heads, max_context_len, stiles) : SharedPlan{};
    const Plan plan = stiles > 0 ? sp.base : plan_decode(d, num_seqs, num_q_heads, max_context_len, partition_size);
    const uint64_t ws_needed = stiles > 0 ? sp.total : plan.ws_total;
    kvp::DecodeArgs a;
    memset(&a, 0, sizeof a);
    if (static_scratch && ws_needed > 0) {
        if (ws_needed > kScratchBytes)
            return fail(KV_ERR_WORKSPACE_TOO_SMALL,
                        "paged_attention_decode_noalloc: this call needs %llu bytes of workspace, the static array "
                        "holds %llu", (unsigned long long)ws_needed, (unsigned long long)kScratchBytes);
        int dev = 0;
        kv_status st = stream_device(stream, &dev);
        if (st != KV_OK) return st;
        st = scratch_on_device(dev, &workspace);
        if (st != KV_OK) return st;
        workspace_bytes = kScratchBytes;
    }
    if (ws_needed > 0) {
        if (!workspace || workspace_bytes < ws_needed)
            return fail(KV_ERR_WORKSPACE_TOO_SMALL, "workspace of %llu bytes given, %llu needed",
                        (unsigned long long)workspace_bytes, (unsigned long long)ws_needed);
        if (!aligned16(workspace)) return fail(KV_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
        char* ws = static_cast<char*>(workspace);
        if (plan.mode == Mode::kBalanced) {
            a.ws_prefix = reinterpret_cast<int64_t*>(ws);
        } else {
            a.ws_ml = reinterpret_cast<float*>(ws);
        }
        a.ws_acc = reinterpret_cast<float*>(ws + plan.ws_first);
        if (stiles > 0) {
            a.ws_pml = reinterpret_cast<float*>(ws + sp.pml_off);
            a.ws_pacc = reinterpret_cast<float*>(ws + sp.pacc_off);
        }
    }
    a.k_layer = pool->k_base + (uint64_t)layer * pool->layer_bytes;
    a.v_layer = pool->v_base + (uint64_t)layer * pool->layer_bytes;
    a.q = q;
    a.out = out;
    a.tables = block_tables;
    a.lens = context_lens;
    a.max_blocks = max_blocks_per_seq;
    a.num_seqs = num_seqs;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = d.num_kv_heads;
    a.num_blocks = d.num_blocks;
    a.block_size = d.block_size;
    a.max_context = max_context_len;
    a.part_tokens = plan.part_tokens;
    a.max_parts = plan.max_parts;
    a.scale_log2 = (float)((double)scale * 1.4426950408889634);   // exp(x) = 2^(x log2 e)
    const bool fp8 = d.dtype == KV_FP8_E4M3;
    if (fp8) {
        a.k_scale = pool->k_scale + (uint64_t)layer * pool->scale_layer;
        a.v_scale = pool->v_scale + (uint64_t)layer * pool->scale_layer;
    }
    hipError_t e;
    if (stiles > 0) {
        a.shared_tiles = stiles;
        a.shared_entries = (int32_t)((int64_t)stiles * kvp::kTileTokens / d.block_size);
        a.prefix_parts = sp.parts;
        a.prefix_part_tiles = sp.part_tiles;
        e = num_rows > 0 ? launch_rows(pool, layer, rows_k, rows_v, rows_slots, num_rows, stream) : hipSuccess;
        if (e == hipSuccess)
            e = kvp::launch_decode_bf16_shared(a, num_q_heads / d.num_kv_heads, plan.workers,
                                               static_cast<hipStream_t>(stream));
    } else if (plan.mode == Mode::kBalanced) {
        // the worker that owns each (sequence, KV head)'s last block uses the new row
        // (FP8: quantized in registers); extra waves of the same launch store it.
        // Other rows are stored by more waves of the launch (FP8: each wave
        // sets the scales of the blocks its rows open).
        a.k_append = k_append;
        a.v_append = v_append;
        e = hipSuccess;
        if (num_rows > 0) {
            a.rows_k = rows_k;
            a.rows_v = rows_v;
            a.rows_slots = rows_slots;
            a.num_rows = num_rows;
        }
        const int group = num_q_heads / d.num_kv_heads;
        if (e == hipSuccess) {
            e = fp8 ? kvp::launch_decode_fp8_streamk(a, group, plan.workers, static_cast<hipStream_t>(stream))
                    : kvp::launch_decode_bf16_streamk(a, group, plan.workers, static_cast<hipStream_t>(stream));
        }
    } else {
        // other rows, then the new rows (FP8: quantized, with the scale of a block they open), then the decode
        e = num_rows > 0 ? launch_rows(pool, layer, rows_k, rows_v, rows_slots, num_rows, stream) : hipSuccess;
        if (append && e == hipSuccess) {
            kvp::AppendArgs w;
            memset(&w, 0, sizeof w);
            w.k_layer = pool->k_base + (uint64_t)layer * pool->layer_bytes;
            w.v_layer = pool->v_base + (uint64_t)layer * pool->layer_bytes;
            w.k_new = k_append;
            w.v_new = v_append;
            w.tables = block_tables;
            w.lens = context_lens;
            w.max_blocks = max_blocks_per_seq;
            w.num_seqs = num_seqs;
            w.num_blocks = d.num_blocks;
            w.max_context = max_context_len;
            w.num_kv_heads = d.num_kv_heads;
            w.row_chunks = d.head_dim * pool->elem_bytes / 16;
            w.block_size = d.block_size;
            if (fp8) {
                w.k_scale = pool->k_scale + (uint64_t)layer * pool->scale_layer;
                w.v_scale = pool->v_scale + (uint64_t)layer * pool->scale_layer;
                e = kvp::launch_append_fp8(w, static_cast<hipStream_t>(stream));
            } else {
                e = kvp::launch_append_scatter(w, static_cast<hipStream_t>(stream));
            }
        }
        if (e == hipSuccess) {
            if (plan.mode == Mode::kPartitions && plan.workers > 0) {
                const int group = num_q_heads / d.num_kv_heads;
                e = fp8 ? kvp::launch_decode_fp8_partitions(a, group, plan.workers, static_cast<hipStream_t>(stream))
                        : kvp::launch_decode_bf16_partitions(a, group, plan.workers, static_cast<hipStream_t>(stream));
                if (e == hipSuccess) e = kvp::launch_partition_merge_bf16(a, static_cast<hipStream_t>(stream));
            } else {
                e = kvp::launch_decode(a, d.dtype, d.head_dim, static_cast<hipStream_t>(stream));
            }
        }
    }
    if (e != hipSuccess) return hip_fail(e, "decode launch");
    return ok();
}

}  // namespace

extern "C" {

kv_status paged_attention_decode(kv_pool_t pool, int32_t layer, void* out, const void* q,
                                 const int32_t* block_tables, int32_t max_blocks_per_seq,
                                 const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads, float scale,
                                 int32_t max_context_len, int32_t partition_size, void* workspace,
                                 uint64_t workspace_bytes, void* stream) {
    return decode_impl(pool, layer, out, q, nullptr, nullptr, block_tables, max_blocks_per_seq, context_lens,
                       num_seqs, num_q_heads, scale, max_context_len, partition_size, workspace, workspace_bytes,
                       stream);
}

kv_status paged_attention_decode_noalloc(kv_pool_t pool, int32_t layer, void* out, const void* q,
                                         const int32_t* block_tables, int32_t max_blocks_per_seq,
                                         const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                                         float scale, int32_t max_context_len, int32_t partition_size,
                                         void* stream) {
    return decode_impl(pool, layer, out, q, nullptr, nullptr, block_tables, max_blocks_per_seq, context_lens,
                       num_seqs, num_q_heads, scale, max_context_len, partition_size, nullptr, 0, stream, 0, true);
}

kv_status paged_attention_decode_shared(kv_pool_t pool, int32_t layer, void* out, const void* q,
                                        const int32_t* block_tables, int32_t max_blocks_per_seq,
                                        const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                                        float scale, int32_t max_context_len, int32_t shared_blocks, void* workspace,
                                        uint64_t workspace_bytes, void* stream) {
    if (shared_blocks < 0) return fail(KV_ERR_INVALID_ARGUMENT, "shared_blocks %d < 0", shared_blocks);
    return decode_impl(pool, layer, out, q, nullptr, nullptr, block_tables, max_blocks_per_seq, context_lens,
                       num_seqs, num_q_heads, scale, max_context_len, 0, workspace, workspace_bytes, stream,
                       shared_blocks);
}

kv_status paged_attention_shared_workspace_bytes(kv_pool_t pool, int32_t num_seqs, int32_t num_q_heads,
                                                 int32_t max_context_len, int32_t max_blocks_per_seq,
                                                 int32_t shared_blocks, uint64_t* bytes) {
    if (!pool || !bytes) return fail(KV_ERR_INVALID_ARGUMENT, "NULL argument");
    *bytes = 0;
    if (num_seqs < 0 || num_q_heads <= 0 || max_context_len < 0 || max_blocks_per_seq <= 0)
        return fail(KV_ERR_INVALID_ARGUMENT, "negative size argument");
    if (num_q_heads % pool->desc.num_kv_heads != 0)
        return fail(KV_ERR_INVALID_ARGUMENT, "num_q_heads %d is not a multiple of num_kv_heads %d", num_q_heads,
                    pool->desc.num_kv_heads);
    const kv_status st = check_shared(pool->desc, num_seqs, max_context_len, max_blocks_per_seq, shared_blocks);
    if (st != KV_OK) return st;
    const int32_t stiles = shared_blocks > 0 ? shared_tiles_of(pool->desc, shared_blocks) : 0;
    *bytes = stiles > 0 ? plan_shared(pool->desc, num_seqs, num_q_heads, max_context_len, stiles).total
                        : plan_decode(pool->desc, num_seqs, num_q_heads, max_context_len, 0).ws_total;
    return ok();
}

kv_status paged_attention_decode_step(kv_pool_t pool, int32_t layer, void* out, const void* q, const void* k_new,
                                      const void* v_new, const int32_t* block_tables, int32_t max_blocks_per_seq,
                                      const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads, float scale,
                                      int32_t max_context_len, int32_t partition_size, const void* k_rows,
                                      const void* v_rows, const int64_t* row_slots, int64_t num_rows, void* workspace,
                                      uint64_t workspace_bytes, void* stream) {
    if (num_seqs > 0 && (!k_new || !v_new)) return fail(KV_ERR_INVALID_ARGUMENT, "k_new/v_new is NULL");
    return decode_impl(pool, layer, out, q, k_new, v_new, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                       num_q_heads, scale, max_context_len, partition_size, workspace, workspace_bytes, stream, 0, false,
                       k_rows, v_rows, row_slots, num_rows);
}

kv_status paged_attention_decode_append(kv_pool_t pool, int32_t layer, void* out, const void* q, const void* k_new,
                                        const void* v_new, const int32_t* block_tables, int32_t max_blocks_per_seq,
                                        const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                                        float scale, int32_t max_context_len, int32_t partition_size,
                                        void* workspace, uint64_t workspace_bytes, void* stream) {
    if (num_seqs > 0 && (!k_new || !v_new)) return fail(KV_ERR_INVALID_ARGUMENT, "k_new/v_new is NULL");
    return decode_impl(pool, layer, out, q, k_new, v_new, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                       num_q_heads, scale, max_context_len, partition_size, workspace, workspace_bytes, stream);
}

}  // extern "C"
