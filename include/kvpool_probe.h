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

#ifdef __cplusplus
}
#endif

#endif /* KVPOOL_PROBE_H */
