/*
 * kvpool_probe.h - measurement probes shipped with libkvpool.so.
 *
 * Not part of the hot path.  They exist so that hardware counters and
 * achieved bandwidth can be read against a kernel whose traffic is known
 * exactly (the copy), and so that the cost of walking block tables can be
 * seen apart from the K/V stream ([KVC] aicassindra.com "GPU paged KV cache",
 * "Inside the paged attention kernel": the per-block cost of the indirection
 * is one integer lookup).
 */
#ifndef KVPOOL_PROBE_H
#define KVPOOL_PROBE_H

#include <stdint.h>

#include "kvpool.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Copy `bytes` bytes from device buffer `src` to device buffer `dst` with 16-byte
 * vector loads and stores: exactly `bytes` read and `bytes` written.  Both
 * pointers 16-byte aligned, bytes a multiple of 16, buffers not overlapping.
 * Queued on `stream` (hipStream_t as void*).  Errors: KV_ERR_INVALID_ARGUMENT,
 * KV_ERR_HIP.
 */
kv_status kv_probe_copy(void* dst, const void* src, uint64_t bytes, void* stream);

/*
 * Read `bytes` bytes of device buffer `src` with 16-byte vector loads and fold
 * them into one 32-bit word per workgroup, written to device buffer `sink`
 * (at least 65536 bytes, 4-byte aligned).  Reads exactly `bytes`; writes at
 * most 64 KiB.  It measures the achievable HBM read rate, and reading a
 * buffer larger than the caches evicts them without leaving dirty lines.
 * src 16-byte aligned, bytes a multiple of 16.  Errors: KV_ERR_INVALID_ARGUMENT,
 * KV_ERR_HIP.
 */
kv_status kv_probe_read(const void* src, uint64_t bytes, void* sink, void* stream);

/*
 * Block-table walk of the balanced decode split (paged_attention_decode with
 * partition_size 0) without the K/V stream: the same workers and slices, the
 * same table-entry loads, no tile loads.  Its L2 hit rate under a counter
 * profiler is the hit rate of the decode's table reads.  xcd_grouped != 0
 * runs slice s on XCD s / (W / 8) instead of XCD s % 8, so the KV heads of a
 * sequence share one XCD.  Arguments as for paged_attention_decode; sink is a
 * device buffer of at least 4 bytes per worker (4096 covers 1024 workers),
 * one folded word per worker is written there.  Errors:
 * KV_ERR_INVALID_ARGUMENT, KV_ERR_HIP.
 */
kv_status kv_probe_table_walk(const int32_t* block_tables, int32_t max_blocks_per_seq,
                              const int32_t* context_lens, int32_t num_seqs, int32_t num_kv_heads,
                              int32_t max_context_len, int32_t xcd_grouped, void* sink, uint64_t sink_bytes,
                              void* stream);

/*
 * The E4M3 conversions of the FP8 pool kernels, one element per call site, so
 * that they can be checked against the format's definition code by code
 * (kv_pool_create_fp8 in kvpool.h describes the format):
 *   kv_probe_e4m3_to_bf16: n codes (device, uint8) -> n bfloat16 bit patterns
 *                          (device, uint16, 2-byte aligned), exact widening;
 *   kv_probe_f32_to_e4m3:  n fp32 values (device, 4-byte aligned) -> n codes,
 *                          round to nearest, ties to the even code, +-448
 *                          saturation, NaN -> 0x7F.
 * Queued on `stream`.  Errors: KV_ERR_INVALID_ARGUMENT, KV_ERR_HIP.
 */
kv_status kv_probe_e4m3_to_bf16(const void* codes, void* out_bf16, int64_t n, void* stream);
kv_status kv_probe_f32_to_e4m3(const float* x, void* out_codes, int64_t n, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVPOOL_PROBE_H */
