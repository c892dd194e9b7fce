// Host-only arithmetic and argument checks of the C-ABI layer: pool and scale
// sizes with overflow checks, and the slot mapping of a step's writes.  Free
// of HIP, so that a host compiler takes it as is: the library includes it,
// and a host-side test builds it with the address and undefined-behaviour
// sanitizers.  Each check returns a kv_status and, on failure, a message in
// the caller's buffer.
#pragma once

#include <stdint.h>
#include <stdio.h>

#include <algorithm>
#include <vector>

#include "kvpool.h"

namespace kvp {
namespace host {

struct Message {
    char text[256];
};

inline kv_status failed(Message& m, kv_status s, const char* text) {
    snprintf(m.text, sizeof m.text, "%s", text);
    return s;
}

inline int elem_bytes_of(int32_t dtype) {
    return dtype == KV_F32 ? 4 : (dtype == KV_BF16 ? 2 : (dtype == KV_FP8_E4M3 ? 1 : 0));
}

inline bool mul_ok(uint64_t a, uint64_t b, uint64_t* out) {
    if (a != 0 && b > UINT64_MAX / a) return false;
    *out = a * b;
    return true;
}

inline kv_status check_desc(const kv_pool_desc* d, Message& m) {
    if (!d) return failed(m, KV_ERR_INVALID_ARGUMENT, "descriptor is NULL");
    if (d->num_layers <= 0 || d->num_blocks <= 0 || d->block_size <= 0 || d->num_kv_heads <= 0 || d->head_dim <= 0) {
        snprintf(m.text, sizeof m.text,
                 "descriptor sizes must be positive (layers %d, blocks %d, block_size %d, kv_heads %d, head_dim %d)",
                 d->num_layers, d->num_blocks, d->block_size, d->num_kv_heads, d->head_dim);
        return KV_ERR_INVALID_ARGUMENT;
    }
    if (elem_bytes_of(d->dtype) == 0) {
        snprintf(m.text, sizeof m.text, "unknown dtype %d", d->dtype);
        return KV_ERR_INVALID_ARGUMENT;
    }
    return KV_OK;
}

// Bytes of the K (or the V) tensor: layers * blocks * block_size * kv_heads * head_dim * element size.
inline kv_status pool_bytes(const kv_pool_desc* d, uint64_t* bytes, Message& m) {
    const kv_status s = check_desc(d, m);
    if (s != KV_OK) return s;
    uint64_t v = (uint64_t)elem_bytes_of(d->dtype);
    if (!mul_ok(v, (uint64_t)d->head_dim, &v) || !mul_ok(v, (uint64_t)d->num_kv_heads, &v) ||
        !mul_ok(v, (uint64_t)d->block_size, &v) || !mul_ok(v, (uint64_t)d->num_blocks, &v) ||
        !mul_ok(v, (uint64_t)d->num_layers, &v))
        return failed(m, KV_ERR_INVALID_ARGUMENT, "pool size overflows 64 bits");
    *bytes = v;
    return KV_OK;
}

// Bytes of the K (or the V) scale tensor of an FP8 pool (one float per layer,
// block and KV head), 0 for other pools.
inline kv_status scale_bytes(const kv_pool_desc* d, uint64_t* bytes, Message& m) {
    *bytes = 0;
    const kv_status s = check_desc(d, m);
    if (s != KV_OK || d->dtype != KV_FP8_E4M3) return s;
    uint64_t v = 4;
    if (!mul_ok(v, (uint64_t)d->num_kv_heads, &v) || !mul_ok(v, (uint64_t)d->num_blocks, &v) ||
        !mul_ok(v, (uint64_t)d->num_layers, &v))
        return failed(m, KV_ERR_INVALID_ARGUMENT, "scale size overflows 64 bits");
    *bytes = v;
    return KV_OK;
}

// Slot mapping of a step's writes ([KVC] "The write path: slot mapping and
// scatter"): request r writes write_count[r] tokens of table row write_seq[r]
// from position write_start[r]; token position p goes to slot
// table[row][p / B] * B + p % B.  Slots are appended in request order.
// With debug_checks, two writes to one slot in the same call (which the
// scatter would resolve in no defined order) are refused as well.
inline kv_status build_slot_mapping(const int32_t* block_tables, int32_t num_rows, int32_t max_blocks_per_seq,
                                    int32_t block_size, int32_t num_blocks, const int32_t* write_seq,
                                    const int32_t* write_start, const int32_t* write_count, int32_t num_requests,
                                    int64_t* slot_mapping, int64_t capacity, int64_t* num_tokens, bool debug_checks,
                                    Message& m) {
    if (!num_tokens) return failed(m, KV_ERR_INVALID_ARGUMENT, "num_tokens is NULL");
    *num_tokens = 0;
    if (num_requests < 0 || num_rows < 0 || max_blocks_per_seq <= 0 || block_size <= 0 || num_blocks <= 0 || capacity < 0)
        return failed(m, KV_ERR_INVALID_ARGUMENT, "negative or zero size argument");
    if (num_requests > 0 && (!block_tables || !write_seq || !write_start || !write_count || (!slot_mapping && capacity > 0)))
        return failed(m, KV_ERR_INVALID_ARGUMENT, "NULL pointer argument");
    int64_t n = 0;
    for (int32_t r = 0; r < num_requests; ++r) {
        const int32_t row = write_seq[r];
        if (row < 0 || row >= num_rows) {
            snprintf(m.text, sizeof m.text, "request %d names row %d of %d", r, row, num_rows);
            return KV_ERR_INVALID_ARGUMENT;
        }
        if (write_start[r] < 0 || write_count[r] < 0) {
            snprintf(m.text, sizeof m.text, "request %d has negative start or count", r);
            return KV_ERR_INVALID_ARGUMENT;
        }
        const int32_t* trow = block_tables + (int64_t)row * max_blocks_per_seq;
        for (int64_t p = write_start[r], e = (int64_t)write_start[r] + write_count[r]; p < e; ++p) {
            const int64_t lb = p / block_size;
            if (lb >= max_blocks_per_seq) {
                snprintf(m.text, sizeof m.text, "request %d position %lld is past its %d-entry table row", r,
                         (long long)p, max_blocks_per_seq);
                return KV_ERR_OUT_OF_RANGE;
            }
            const int32_t phys = trow[lb];
            if (phys < 0 || phys >= num_blocks) {
                snprintf(m.text, sizeof m.text, "row %d entry %lld = %d is outside the %d-block pool", row,
                         (long long)lb, phys, num_blocks);
                return KV_ERR_OUT_OF_RANGE;
            }
            if (n >= capacity) {
                snprintf(m.text, sizeof m.text, "slot_mapping capacity %lld too small", (long long)capacity);
                return KV_ERR_INVALID_ARGUMENT;
            }
            slot_mapping[n++] = (int64_t)phys * block_size + (p - lb * block_size);
        }
    }
    if (debug_checks && n > 1) {
        std::vector<int64_t> sorted(slot_mapping, slot_mapping + n);
        std::sort(sorted.begin(), sorted.end());
        const auto dup = std::adjacent_find(sorted.begin(), sorted.end());
        if (dup != sorted.end()) {
            snprintf(m.text, sizeof m.text, "slot %lld is written twice in one call", (long long)*dup);
            return KV_ERR_INVALID_ARGUMENT;
        }
    }
    *num_tokens = n;
    return KV_OK;
}

}  // namespace host
}  // namespace kvp
