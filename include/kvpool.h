/*
 * kvpool.h - C ABI of the MI355X (gfx950) paged KV-cache hot path.
 *
 * Two device steps and the host step that feeds them:
 *   - kv_build_slot_mapping   (host)  turns each sequence's block table and the
 *                                     positions written this step into one
 *                                     linear slot per token;
 *   - reshape_and_cache       (GPU)   scatters the new tokens' K and V into the
 *                                     block pool through that slot mapping;
 *   - paged_attention_decode  (GPU)   one query token per sequence attends over
 *                                     its whole context, reading K and V through
 *                                     the sequence's block table (grouped-query
 *                                     attention, online softmax, optional split
 *                                     of the context into partitions merged by
 *                                     a second kernel).
 * Beside them: the decode append folded into the attention call, the
 * copy-on-write block copy, FP8 pools with per-block scales, and swap of
 * blocks to pinned host memory and back.
 *
 * Sources (page title, section):
 *   [KVC] aicassindra.com "GPU paged KV cache":
 *         "Fixed-size blocks and the block-table indirection" (blocks of B
 *         tokens, table entry i names the physical block of tokens
 *         [i*B, (i+1)*B), one 32-bit index per block);
 *         "Sizing the pool" (pool preallocated once, one K and one V tensor per
 *         layer; per-token cost 2 * kv_heads * head_dim * bytes per layer);
 *         "The write path: slot mapping and scatter" (one integer per token,
 *         block_index * B + offset, built on the host each step; tables at a
 *         fixed address, updated in place, for graph replay; head_dim
 *         innermost and contiguous);
 *         "Inside the paged attention kernel" (per (sequence, KV head) walk of
 *         logical blocks through the table, online softmax, split of long
 *         contexts over several workgroups merged by a cheap reduction).
 *   [PIF] "PagedAttention, Internals First", "02 Block tables" (token t in
 *         logical block t / B at offset t % B; each KV head serves its group of
 *         query heads).
 *   [TMP] aicassindra.com transformer-math "paged attention", "End-to-end
 *         flow" (the step attends over the full history including the token
 *         written this step).
 *   [LAT] lattice-ai-eng "KV Cache & PagedAttention", "5. Production
 *         tradeoffs" (an FP8 cache halves cache memory and decode traffic).
 *
 * Conventions for every call:
 *   - Device pointers are borrowed: the caller allocates them and keeps them
 *     alive until the work queued on `stream` has finished.  The library never
 *     allocates device memory at run time and never synchronises (its one
 *     static device array, the workspace of paged_attention_decode_noalloc,
 *     is part of the loaded code object).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work
 *     is queued and the call returns; results are ordered by the stream.
 *   - Host-checkable argument errors return a negative kv_status before any
 *     launch; kv_last_error_message() then holds a readable detail (per thread).
 *   - Device-side data (slot mappings, tables, lengths) is trusted but bounded:
 *     kernels never read or write outside the pool, the tables or the outputs
 *     whatever those values are; values that break the preconditions give an
 *     unspecified result for the tokens or sequences concerned.
 *
 * Pool layout, per layer, for both the K and the V tensor:
 *     [num_blocks][num_kv_heads][block_size][head_dim]      (head_dim innermost)
 * and layers follow each other: layer l starts at base + l * (bytes of one layer).
 * One (block, KV head) tile is block_size * head_dim contiguous elements.
 */
#ifndef KVPOOL_H
#define KVPOOL_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kv_status {
    KV_OK = 0,
    KV_ERR_INVALID_ARGUMENT = -1,   /* null or misaligned pointer, bad size, bad index */
    KV_ERR_UNSUPPORTED = -2,        /* valid but not built: dtype, head_dim, block size, group size */
    KV_ERR_WORKSPACE_TOO_SMALL = -3,
    KV_ERR_HIP = -4,                /* the HIP runtime reported an error at launch */
    KV_ERR_OUT_OF_RANGE = -5        /* host-side table entry or position outside the pool or the table */
} kv_status;

typedef enum kv_dtype {
    KV_F32 = 0,      /* IEEE binary32 */
    KV_BF16 = 1,     /* bfloat16 (upper half of binary32); fp32 accumulation, round-to-nearest-even stores */
    KV_FP8_E4M3 = 2  /* pool holds OCP E4M3 codes (1 sign, 4 exponent bits with bias 7, 3 mantissa bits,
                      * largest finite 448, 0x7F/0xFF NaN) with one fp32 scale per (block, KV head) for K
                      * and one for V; a stored value is code * scale.  q, k_new/v_new and the output
                      * are bf16.  head_dim 128, block_size 8, 16, 32, 64 or 128. */
} kv_dtype;

typedef struct kv_pool_desc {
    int32_t num_layers;     /* >= 1 */
    int32_t num_blocks;     /* physical blocks per layer, >= 1 */
    int32_t block_size;     /* tokens per block (B): 16; bf16 pools with head_dim 128 also 8, 32, 64, 128 */
    int32_t num_kv_heads;   /* KV heads per layer */
    int32_t head_dim;       /* elements per head row; the kernels are built for 64 and 128 */
    int32_t dtype;          /* kv_dtype of the pool; q, k_new/v_new and the output are in it too
                             * (bf16 for KV_FP8_E4M3) */
} kv_pool_desc;

/* Opaque host-side handle: the descriptor and the two base pointers.  Immutable
 * after creation, so one handle may be used from several threads at once. */
typedef struct kv_pool* kv_pool_t;

/*
 * Bytes of ONE of the two pool tensors (K or V), all layers:
 *     num_layers * num_blocks * block_size * num_kv_heads * head_dim * elem_bytes
 * [KVC "Sizing the pool"].  Pure arithmetic: accepts any positive sizes, also
 * ones the kernels are not built for.  Errors: KV_ERR_INVALID_ARGUMENT for a
 * null pointer, a non-positive size, an unknown dtype or a 64-bit overflow.
 */
kv_status kv_pool_bytes(const kv_pool_desc* desc, uint64_t* bytes_per_tensor);

/*
 * Wrap two caller-allocated device buffers of kv_pool_bytes() bytes each as a
 * pool.  No device memory is allocated or touched.  k_base and v_base must be
 * 16-byte aligned.  Errors: KV_ERR_INVALID_ARGUMENT (null, misaligned, bad
 * descriptor, an FP8 dtype: see kv_pool_create_fp8), KV_ERR_UNSUPPORTED
 * (head_dim not 64 or 128; block_size not 16, or for bf16 pools with head_dim
 * 128 not one of 8, 16, 32, 64, 128).
 */
kv_status kv_pool_create(const kv_pool_desc* desc, void* k_base, void* v_base, kv_pool_t* out);

/*
 * FP8 pools (KV_FP8_E4M3): blocks as quantization groups ([PIF] "06 Open
 * questions": per-block scales ride along with the block, CoW copies included;
 * [LAT] "5. Production tradeoffs", Quality: FP8 KV halves cache bytes and
 * decode traffic).  Besides the two code tensors (kv_pool_bytes each, one byte
 * per element), a pool has two scale tensors, fp32
 * [num_layers][num_blocks][num_kv_heads], of kv_pool_scale_bytes bytes each.
 * Scales travel with their block: kv_copy_blocks copies them.  The write that
 * covers row 0 of a block sets that block's scales to amax / 448 over the rows
 * it puts there (1.0 when all are zero); later writes into the block keep the
 * scales and saturate at +-448, so a block is never requantized.  Quantizing
 * is fp32 division by the scale, then round to the nearest E4M3 value, ties to
 * the even code.
 */
kv_status kv_pool_scale_bytes(const kv_pool_desc* desc, uint64_t* bytes_per_tensor);   /* 0 unless FP8 */

/*
 * kv_pool_create for KV_FP8_E4M3: also wraps the two caller-allocated scale
 * tensors (4-byte aligned).  Errors: as kv_pool_create; KV_ERR_INVALID_ARGUMENT
 * when the dtype is not KV_FP8_E4M3 or a scale pointer is null or misaligned;
 * KV_ERR_UNSUPPORTED unless head_dim is 128 and block_size one of 8, 16, 32,
 * 64, 128.
 */
kv_status kv_pool_create_fp8(const kv_pool_desc* desc, void* k_codes, void* v_codes, float* k_scales,
                             float* v_scales, kv_pool_t* out);

/* Free the handle (not the buffers).  NULL is accepted. */
kv_status kv_pool_destroy(kv_pool_t pool);

/*
 * Host step [KVC "The write path"; PIF "02 Block tables"]: for each request r
 * and each logical position p in [write_start[r], write_start[r] + write_count[r]),
 * in request order, emit
 *     slot = block_tables[write_seq[r]][p / B] * B + p % B.
 * All pointers are HOST pointers.  block_tables is int32 [num_rows][max_blocks_per_seq],
 * row-major.  On success *num_tokens holds the number of slots written to
 * slot_mapping (capacity entries available).  Errors: KV_ERR_INVALID_ARGUMENT
 * (null pointer, negative count or start, row outside [0, num_rows), capacity
 * too small), KV_ERR_OUT_OF_RANGE (p / B >= max_blocks_per_seq, or a table
 * entry outside [0, num_blocks)).  Nothing is written past the first error.
 * A library built with KV_DEBUG (python -m paged_kv_cache_num_amd.build --debug)
 * also refuses, with KV_ERR_INVALID_ARGUMENT, two writes to one slot in the same
 * call (the scatter would apply them in no defined order); *num_tokens is then 0.
 */
kv_status kv_build_slot_mapping(const int32_t* block_tables, int32_t num_rows,
                                int32_t max_blocks_per_seq, int32_t block_size, int32_t num_blocks,
                                const int32_t* write_seq, const int32_t* write_start,
                                const int32_t* write_count, int32_t num_requests,
                                int64_t* slot_mapping, int64_t capacity, int64_t* num_tokens);

/*
 * GPU step [KVC "The write path: slot mapping and scatter"]: for every token t
 * with 0 <= slot_mapping[t] < num_blocks * B, copy the bits of k_new[t][h][:]
 * and v_new[t][h][:] to row (slot / B, h, slot % B) of layer `layer` of the K
 * and V pools, for every KV head h.  Tokens with a negative slot (padding) or a
 * slot past the pool are skipped.  A bit-exact copy.
 * FP8 pools: k_new / v_new are bf16; first every block whose row 0 one of the
 * tokens writes gets its K and V scales (per KV head) from the rows this call
 * puts into that block, then every row is quantized with its block's scale
 * (the rule under kv_pool_scale_bytes).  Rows should be finite (a NaN or an
 * infinity gives an unspecified result for its block).  Two kernels in
 * stream order.
 *   k_new, v_new:   device, [num_tokens][num_kv_heads][head_dim], pool dtype (bf16 for FP8), 16-byte aligned
 *   slot_mapping:   device, int64 [num_tokens]
 * Precondition: non-negative slots are unique (two tokens for one slot race).
 * num_tokens == 0 queues nothing.  Errors: KV_ERR_INVALID_ARGUMENT (null
 * handle or pointer, misalignment, layer out of range, num_tokens < 0),
 * KV_ERR_UNSUPPORTED (num_kv_heads above 2^20), KV_ERR_HIP.
 */
kv_status reshape_and_cache(kv_pool_t pool, int32_t layer, const void* k_new, const void* v_new,
                            const int64_t* slot_mapping, int64_t num_tokens, void* stream);

/*
 * GPU step, copy-on-write ([KVC] "Prefix sharing, reference counts, and
 * copy-on-write"; [PIF] "03 Sharing via copy-on-write"): before a sequence
 * writes into a block that other tables also name, the block manager takes a
 * fresh block, has its contents copied, and repoints the writer's table entry.
 * This call is that device copy: for every pair p, block block_pairs[2p] is
 * copied to block block_pairs[2p + 1] in every layer of the K and the V tensor
 * (H_kv * B * D * e contiguous bytes per layer and tensor), bit for bit; in an
 * FP8 pool the block's K and V scales of every layer are copied too.
 *   block_pairs: device, int32 [num_pairs][2] (src, dst), 4-byte aligned.
 *                A pair naming a block outside [0, num_blocks) is skipped.
 *   Precondition: no destination appears twice or as a source of another
 *   pair (the copies run in no particular order).
 * The refcount check and the table update are host bookkeeping of the block
 * manager; the library does not keep reference counts.
 * Errors: KV_ERR_INVALID_ARGUMENT (null handle, negative count, null or
 * misaligned pairs), KV_ERR_HIP.  num_pairs == 0 queues nothing.
 */
kv_status kv_copy_blocks(kv_pool_t pool, const int32_t* block_pairs, int32_t num_pairs, void* stream);

/*
 * Swap to and from host memory ([KVC] "Reclaiming memory: swap versus
 * recompute": a preempted sequence's blocks are copied to pinned host memory
 * and back on resume, twice its KV bytes over the host link; [PIF] "05
 * Preemption and the scheduler contract").  Freeing the blocks in between and
 * choosing victims is the block manager's host bookkeeping, not done here.
 *
 * The host buffer holds one record of kv_swap_bytes(pool, 1, ...) bytes per
 * listed block, in list order: for each layer, the block's K run then its V
 * run (H_kv * B * D * e bytes each, the pool's bytes unchanged); for FP8 pools
 * then, for each layer, the block's K scales then its V scales (H_kv fp32
 * each); zero padding to a multiple of 16 bytes.
 *
 *   kv_swap_bytes: host bytes for num_blocks blocks (num_blocks >= 0).
 *   kv_swap_out:   GPU step: copy blocks[i] (device int32 list, 4-byte aligned)
 *                  of every layer to record i of host_buf.
 *   kv_swap_in:    GPU step: copy record i of host_buf to block blocks[i] of
 *                  every layer (the blocks may differ from those swapped out;
 *                  the caller then repoints the table entries).
 * host_buf must be pinned host memory that the device can address
 * (hipHostMalloc; torch's pin_memory), 16-byte aligned, with host_bytes at
 * least kv_swap_bytes(pool, num_blocks); the kernels read and write it
 * directly over the host link, one launch per call, and the caller keeps it
 * alive until the stream has passed the call.  A list entry outside
 * [0, num_blocks) is skipped (its record is left as it was, or not read).
 * Precondition for kv_swap_in: no block listed twice.  Bit-exact both ways.
 * Errors: KV_ERR_INVALID_ARGUMENT (null or misaligned pointer, negative count,
 * host buffer too small, not pinned or without a device mapping), KV_ERR_HIP.
 * num_blocks == 0 queues nothing.
 */
kv_status kv_swap_bytes(kv_pool_t pool, int32_t num_blocks, uint64_t* bytes);
kv_status kv_swap_out(kv_pool_t pool, const int32_t* blocks, int32_t num_blocks, void* host_buf,
                      uint64_t host_bytes, void* stream);
kv_status kv_swap_in(kv_pool_t pool, const int32_t* blocks, int32_t num_blocks, const void* host_buf,
                     uint64_t host_bytes, void* stream);

/*
 * Workspace needed by paged_attention_decode for this shape and mode (see
 * partition_size below).  Zero when no workspace is used.  With partitions it
 * holds one fp32 running max, sum and unnormalised output per (sequence,
 * query head, partition); in the balanced mode, the tiles before each
 * sequence (int64, num_seqs + 1) and at most two fp32 partial states per
 * worker (one worker wave per SIMD for bf16 pools, two for FP8 pools, at
 * most 2048).  The balanced-mode size depends on the current device's
 * compute unit count: query it on the device that will run the call.
 * Errors: KV_ERR_INVALID_ARGUMENT (null, negative sizes, partition_size not a
 * multiple of the block size, num_q_heads not a multiple of num_kv_heads).
 */
kv_status paged_attention_workspace_bytes(kv_pool_t pool, int32_t num_seqs, int32_t num_q_heads,
                                          int32_t max_context_len, int32_t partition_size,
                                          uint64_t* bytes);

/*
 * GPU step [KVC "Inside the paged attention kernel"; PIF "02 Block tables";
 * TMP "End-to-end flow"]: for every sequence i and query head h, with
 * g = num_q_heads / num_kv_heads and kv = h / g,
 *     out[i][h][:] = sum_j softmax_j(scale * q[i][h] . K_i[j]) V_i[j],
 * j over the first L_i = context_lens[i] logical tokens of sequence i, where
 * K_i[j] / V_i[j] are row (block_tables[i][j / B], kv, j % B) of layer `layer`.
 * L_i counts the token written this step.  L_i == 0 gives a zero output.
 * FP8 pools: K_i[j] and V_i[j] are the codes times their block's K / V scale
 * for head kv; q and out are bf16.
 *   out, q:        device, [num_seqs][num_q_heads][head_dim], pool dtype (bf16 for FP8), 16-byte aligned
 *   block_tables:  device, int32 [num_seqs][max_blocks_per_seq]; entries at
 *                  b >= ceil(L_i / B) are never read
 *   context_lens:  device, int32 [num_seqs], each in [0, max_context_len]
 *   max_context_len: host bound on every L_i (sizes the grid); <= max_blocks_per_seq * B
 *   partition_size: 0 = the library balances the work itself.  For bf16 and FP8
 *                  pools with head_dim 128 and at most 1024 sequences, the
 *                  (sequence, KV head, block) tiles of the whole batch are cut
 *                  into equal contiguous slices, one per resident wave, and
 *                  a second kernel merges the (sequence, KV head) pairs that
 *                  straddle slices; other shapes walk each context in one
 *                  workgroup per (sequence, KV head).
 *                  > 0: a multiple of B; each context is cut into partitions
 *                  of that many tokens, each computed whole by one wave (for
 *                  bf16 and FP8 pools with head_dim 128 and at most 1024
 *                  sequences the partitions of the whole batch are shared out
 *                  to one resident wave per SIMD; otherwise one workgroup per
 *                  partition), and a second kernel merges them (log-sum-exp
 *                  rescale).
 *   scale:         softmax scale, finite and > 0
 *   workspace:     device, >= paged_attention_workspace_bytes(...) bytes, 16-byte
 *                  aligned; may be NULL when that size is 0.  Its contents on
 *                  entry do not matter.
 * Results do not depend on where blocks live: two tables naming different
 * physical blocks with the same contents give bitwise equal outputs.
 * Errors: KV_ERR_INVALID_ARGUMENT, KV_ERR_UNSUPPORTED (group size not in
 * {1, 2, 4, 8}), KV_ERR_WORKSPACE_TOO_SMALL, KV_ERR_HIP.
 */
kv_status paged_attention_decode(kv_pool_t pool, int32_t layer, void* out, const void* q,
                                 const int32_t* block_tables, int32_t max_blocks_per_seq,
                                 const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                                 float scale, int32_t max_context_len, int32_t partition_size,
                                 void* workspace, uint64_t workspace_bytes, void* stream);

/*
 * GPU step: the decode append and the attention of one step in one call.  The
 * result, pool included, is bitwise that of reshape_and_cache of sequence i's
 * new row to position L_i - 1 (slot table[i][(L_i - 1) / B] * B + (L_i - 1) % B,
 * [KVC] "The write path: slot mapping and scatter") for every i with L_i > 0,
 * followed by paged_attention_decode with the same arguments.
 *   k_new, v_new: device, [num_seqs][H_kv][D] in the pool dtype (bf16 for FP8), 16-byte aligned:
 *                 the K/V row of the token each sequence writes this step
 *                 (rows of sequences with L_i = 0 are not read).
 *   Every other argument, and every error, as for paged_attention_decode.
 * Precondition: the block holding position L_i - 1 of sequence i is named by no
 * other sequence of the call (the block being appended to is private, as after
 * copy-on-write).  In the balanced mode the wave that reads that block writes
 * the row into the pool and uses it directly (one kernel, no separate scatter);
 * other modes run a small scatter kernel first.  A block index outside the pool
 * is skipped, as by reshape_and_cache.  FP8 pools: the row is quantized (a row
 * at position 0 of its block sets that block's scales from itself alone); in
 * the balanced mode the wave that walks the sequence's last tile of a KV head
 * stores that head's row, other modes run a small append kernel first.
 */
kv_status paged_attention_decode_append(kv_pool_t pool, int32_t layer, void* out, const void* q,
                                        const void* k_new, const void* v_new, const int32_t* block_tables,
                                        int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                                        int32_t num_q_heads, float scale, int32_t max_context_len,
                                        int32_t partition_size, void* workspace, uint64_t workspace_bytes,
                                        void* stream);

/*
 * GPU step with other rows: reshape_and_cache(pool, layer, k_rows, v_rows,
 * row_slots, num_rows) followed by paged_attention_decode_append with the
 * remaining arguments, in one call; the result, pool included, is bitwise
 * that of the two calls.  The other rows are those of tokens that this step's
 * attention does not read, such as a prefill chunk of a sequence outside the
 * decode batch ([KVC] "The write path: slot mapping and scatter").
 *   k_rows, v_rows: device, [num_rows][H_kv][D] in the pool dtype (bf16 for FP8), 16-byte aligned.
 *   row_slots:      device, int64 [num_rows], 8-byte aligned; a slot < 0 or >= N * B is skipped.
 *   num_rows:       host, >= 0; 0 makes this paged_attention_decode_append.
 *   Every other argument, and every error, as for paged_attention_decode_append;
 *   with num_seqs = 0 only the rows are stored.
 * Precondition: no slot of row_slots lies in a block that the attention reads
 * (named by sequence i's table within its first L_i positions) or that a
 * decode row is appended to.  In the balanced mode the rows are stored by
 * extra waves of the attention's launch (one kernel, then the fix-up): for a
 * bf16 pool each lane moves several 16-byte chunks; for an FP8 pool a wave
 * takes sixteen rows of one KV head, sets the scales of the blocks whose row 0
 * they hold from every row this call puts into those blocks and stores those
 * blocks' codes, and quantizes any other row with its block's stored scale.
 * In the other modes the scatter kernels run first.
 */
kv_status paged_attention_decode_step(kv_pool_t pool, int32_t layer, void* out, const void* q, const void* k_new,
                                      const void* v_new, const int32_t* block_tables, int32_t max_blocks_per_seq,
                                      const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads, float scale,
                                      int32_t max_context_len, int32_t partition_size, const void* k_rows,
                                      const void* v_rows, const int64_t* row_slots, int64_t num_rows, void* workspace,
                                      uint64_t workspace_bytes, void* stream);

/*
 * GPU step, a batch with a common prefix ([KVC] "Prefix sharing, reference
 * counts, and copy-on-write"; [PIF] "03 Sharing via copy-on-write"): the same
 * result as paged_attention_decode with partition_size 0, up to rounding
 * order, when the first shared_blocks entries of every sequence's table name
 * the same blocks (the block manager's shared, reference-counted prompt).
 * Each (block, KV head) tile of that prefix is then read once for up to
 * sixteen query heads of several sequences together, instead of once per
 * sequence, by extra waves of the balanced split's launch; the rest of each
 * context goes through the balanced split; a second kernel merges the two.
 *   shared_blocks: host, >= 0; 0 runs paged_attention_decode with
 *                  partition_size 0.  shared_blocks * B <= max_context_len and
 *                  <= max_blocks_per_seq * B.
 *   workspace:     device, >= paged_attention_shared_workspace_bytes(...)
 *                  bytes, 16-byte aligned; contents on entry do not matter.
 *   Every other argument as for paged_attention_decode.
 * Preconditions (device data, not checked): block_tables[i][b] ==
 * block_tables[0][b] for every i and b < shared_blocks, and L_i >=
 * shared_blocks * B for every i (a sequence with L_i == 0 still gives zeros).
 * The prefix is read through sequence 0's table row, in whole 16-token tiles
 * (with 8-token blocks an odd last prefix block is read per sequence, as the
 * rest of the context is; a prefix of one 8-token block runs the plain call).
 * Built for bf16 pools with head_dim 128, block sizes 8 to 128, and at most
 * 1024 sequences (KV_ERR_UNSUPPORTED otherwise); no decode-append form.  Errors as for
 * paged_attention_decode.
 */
kv_status paged_attention_decode_shared(kv_pool_t pool, int32_t layer, void* out, const void* q,
                                        const int32_t* block_tables, int32_t max_blocks_per_seq,
                                        const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                                        float scale, int32_t max_context_len, int32_t shared_blocks,
                                        void* workspace, uint64_t workspace_bytes, void* stream);

/*
 * Host: workspace bytes paged_attention_decode_shared needs for these sizes
 * (shared_blocks 0: those of paged_attention_decode with partition_size 0).
 * Errors: KV_ERR_INVALID_ARGUMENT, KV_ERR_UNSUPPORTED, as for the call.
 */
kv_status paged_attention_shared_workspace_bytes(kv_pool_t pool, int32_t num_seqs, int32_t num_q_heads,
                                                 int32_t max_context_len, int32_t max_blocks_per_seq,
                                                 int32_t shared_blocks, uint64_t* bytes);

/*
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * result as paged_attention_decode (bitwise: the same kernels), with the
 * workspace taken from a static device array of KV_NOALLOC_SCRATCH_BYTES
 * bytes that the library holds on every GPU it runs on until the process ends.
 * The call allocates and frees nothing.
 *   Every argument as for paged_attention_decode, less the workspace.  The
 *   device is the stream's (the current device for the NULL stream); the
 *   first call on a device looks up that device's copy of the array.
 *   Calls on one GPU share its array: calls that overlap in time on that GPU
 *   (other streams, other host threads) race, and must be ordered by the
 *   caller.  Nothing in the array needs to hold a given value on entry.
 * Errors: as for paged_attention_decode; KV_ERR_WORKSPACE_TOO_SMALL when the
 * call needs more than KV_NOALLOC_SCRATCH_BYTES of workspace
 * (paged_attention_workspace_bytes tells); KV_ERR_HIP when the array cannot
 * be looked up on the stream's device.
 */
#define KV_NOALLOC_SCRATCH_BYTES (64ull << 20)
kv_status paged_attention_decode_noalloc(kv_pool_t pool, int32_t layer, void* out, const void* q,
                                         const int32_t* block_tables, int32_t max_blocks_per_seq,
                                         const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                                         float scale, int32_t max_context_len, int32_t partition_size,
                                         void* stream);

/* Static name of a status code ("KV_OK", ...); never NULL. */
const char* kv_status_string(kv_status status);

/* Detail of the last failed call on this thread ("" if none); valid until the
 * next call on this thread. */
const char* kv_last_error_message(void);

#ifdef __cplusplus
}
#endif

#endif /* KVPOOL_H */
