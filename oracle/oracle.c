/*
 * CPU oracle for the paged KV-cache hot path: plain, slow, fp64.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file: only the tests, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, constant or helper with
 * the HIP library; it is written from the pages' description of what the path
 * computes, not from the kernels.
 *
 * Sources (page title, section):
 *   [KVC]  aicassindra.com "GPU paged KV cache" blog page
 *          - "Fixed-size blocks and the block-table indirection": a block holds
 *            K and V of B consecutive tokens; table entry i names the physical
 *            block of logical tokens [i*B, (i+1)*B).
 *          - "Sizing the pool": one K and one V tensor per layer.
 *          - "The write path: slot mapping and scatter": one integer per token,
 *            the linear destination block_index * B + offset; head_dim
 *            innermost and contiguous.
 *          - "Inside the paged attention kernel": per (sequence, KV head) walk
 *            the logical blocks, read the physical index from the table, form
 *            q.k dot products, softmax, weighted sum of values.
 *   [PIF]  "PagedAttention, Internals First", "02 Block tables": token t lives
 *          in logical block t // B at offset t % B; the physical location is
 *          block_table[t // B] plus the offset; each KV head serves its group
 *          of query heads.
 *   [TMP]  aicassindra.com transformer-math "paged attention" page, "End-to-end
 *          flow": the decode step attends over the full history including the
 *          token just written; "The architecture: every piece explained":
 *          paging is invisible to the math.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - the softmax scale is an argument (tests pass 1/sqrt(head_dim));
 *   - query head h uses KV head h / (num_q_heads / num_kv_heads);
 *   - a negative slot is skipped; a context length of 0 gives a zero output;
 *   - attention is the two-pass textbook softmax (max, then normalised sum)
 *     over the gathered contiguous K/V, deliberately not an online recurrence.
 *
 * Pool layout, per layer: [num_blocks][num_kv_heads][block_size][head_dim].
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1 };

/* ---- element access -------------------------------------------------- */

/* bfloat16 is the upper half of an IEEE binary32; widening is exact. */
static double bf16_bits_to_double(uint16_t bits) {
    uint32_t w = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

static double load_elem(const void* base, int dtype, int64_t index) {
    if (dtype == ORACLE_F32) return (double)((const float*)base)[index];
    return bf16_bits_to_double(((const uint16_t*)base)[index]);
}

/* Element index of (block, head, offset-in-block, dim) in one layer's pool. */
static int64_t pool_index(int64_t block, int32_t head, int32_t offset, int32_t dim,
                          int32_t num_kv_heads, int32_t block_size, int32_t head_dim) {
    return ((block * num_kv_heads + head) * (int64_t)block_size + offset) * head_dim + dim;
}

/* ---- slot mapping [KVC write path; PIF 02] ----------------------------- */

/*
 * For every write request r (a table row, a first logical position and a
 * token count) and every position p in [start, start+count): the logical
 * block is p / B, the offset p % B, the physical block table[row][p / B],
 * and the slot is physical_block * B + offset.  Tokens are numbered in request
 * order.  Returns the number of slots written, or -1 if a request reaches past
 * its table row, names a row that does not exist, or a table entry is outside
 * [0, num_blocks).
 */
int64_t oracle_slot_mapping(const int32_t* tables, int32_t num_rows, int32_t max_blocks_per_seq,
                            int32_t block_size, int64_t num_blocks,
                            const int32_t* write_seq, const int32_t* write_start,
                            const int32_t* write_count, int32_t num_requests,
                            int64_t* slots, int64_t capacity) {
    int64_t t = 0;
    for (int32_t r = 0; r < num_requests; ++r) {
        int32_t row = write_seq[r];
        if (row < 0 || row >= num_rows || write_start[r] < 0 || write_count[r] < 0) return -1;
        for (int32_t k = 0; k < write_count[r]; ++k) {
            int64_t pos = (int64_t)write_start[r] + k;
            int64_t logical_block = pos / block_size;
            int64_t offset = pos % block_size;
            if (logical_block >= max_blocks_per_seq) return -1;
            int64_t phys = tables[(int64_t)row * max_blocks_per_seq + logical_block];
            if (phys < 0 || phys >= num_blocks) return -1;
            if (t >= capacity) return -1;
            slots[t++] = phys * block_size + offset;
        }
    }
    return t;
}

/* ---- scatter [KVC write path] ------------------------------------------ */

/*
 * For tokens t in order, with slot s = slot_mapping[t] >= 0: block s / B,
 * offset s % B; copy the bytes of k_new[t][h][:] and v_new[t][h][:] into
 * that (block, h, offset) row of the pools for every KV head h.  A plain
 * byte copy: the pool receives exactly the input bits.  Returns 0, or -1 if a
 * slot lies outside the pool (nothing past that token is written).
 */
int oracle_scatter(uint8_t* k_pool, uint8_t* v_pool, int64_t num_blocks, int32_t num_kv_heads,
                   int32_t block_size, int32_t head_dim, int32_t elem_bytes,
                   const uint8_t* k_new, const uint8_t* v_new,
                   const int64_t* slot_mapping, int64_t num_tokens) {
    const int64_t row_bytes = (int64_t)head_dim * elem_bytes;
    for (int64_t t = 0; t < num_tokens; ++t) {
        int64_t s = slot_mapping[t];
        if (s < 0) continue;
        int64_t block = s / block_size;
        int32_t offset = (int32_t)(s % block_size);
        if (block >= num_blocks) return -1;
        for (int32_t h = 0; h < num_kv_heads; ++h) {
            int64_t dst = pool_index(block, h, offset, 0, num_kv_heads, block_size, head_dim) * elem_bytes;
            int64_t src = ((t * num_kv_heads) + h) * row_bytes;
            memcpy(k_pool + dst, k_new + src, (size_t)row_bytes);
            memcpy(v_pool + dst, v_new + src, (size_t)row_bytes);
        }
    }
    return 0;
}

/* ---- paged decode attention [KVC kernel; PIF 02; TMP] ------------------- */

typedef struct {
    double* out;                 /* [num_seqs][num_q_heads][head_dim] */
    const void* q;               /* [num_seqs][num_q_heads][head_dim], storage dtype */
    const void* k_pool;
    const void* v_pool;
    int dtype;
    int64_t num_blocks;
    int32_t num_kv_heads, block_size, head_dim, num_q_heads;
    const int32_t* tables;
    int32_t max_blocks_per_seq;
    const int32_t* context_lens;
    int32_t num_seqs;
    double scale;
    int32_t num_threads;
    int32_t thread_id;
    int status;
} attn_job;

/* One (sequence, KV head) pair: gather, then per query head of the group a
 * two-pass softmax and a weighted sum of the gathered values. */
static int attend_one(const attn_job* J, int32_t seq, int32_t kv) {
    const int32_t D = J->head_dim, B = J->block_size;
    const int32_t group = J->num_q_heads / J->num_kv_heads;
    const int32_t L = J->context_lens[seq];
    if (L < 0 || L > (int64_t)J->max_blocks_per_seq * B) return -1;

    /* 1. gather this sequence's K and V for this head into contiguous rows */
    double* Kc = (double*)malloc(sizeof(double) * ((size_t)L * D + 1));
    double* Vc = (double*)malloc(sizeof(double) * ((size_t)L * D + 1));
    double* w = (double*)malloc(sizeof(double) * ((size_t)L + 1));
    double* qh = (double*)malloc(sizeof(double) * (size_t)D);
    if (!Kc || !Vc || !w || !qh) { free(Kc); free(Vc); free(w); free(qh); return -2; }
    for (int32_t j = 0; j < L; ++j) {
        int64_t phys = J->tables[(int64_t)seq * J->max_blocks_per_seq + j / B];
        if (phys < 0 || phys >= J->num_blocks) { free(Kc); free(Vc); free(w); free(qh); return -1; }
        for (int32_t d = 0; d < D; ++d) {
            int64_t idx = pool_index(phys, kv, j % B, d, J->num_kv_heads, B, D);
            Kc[(int64_t)j * D + d] = load_elem(J->k_pool, J->dtype, idx);
            Vc[(int64_t)j * D + d] = load_elem(J->v_pool, J->dtype, idx);
        }
    }

    /* 2. every query head h with h / group == kv */
    for (int32_t h = kv * group; h < (kv + 1) * group; ++h) {
        double* o = J->out + ((int64_t)seq * J->num_q_heads + h) * D;
        int64_t qbase = ((int64_t)seq * J->num_q_heads + h) * D;
        if (L == 0) {
            for (int32_t d = 0; d < D; ++d) o[d] = 0.0;
            continue;
        }
        for (int32_t d = 0; d < D; ++d) qh[d] = load_elem(J->q, J->dtype, qbase + d);
        double m = -INFINITY;
        for (int32_t j = 0; j < L; ++j) {
            double s = 0.0;
            for (int32_t d = 0; d < D; ++d) s += qh[d] * Kc[(int64_t)j * D + d];
            w[j] = J->scale * s;
            if (w[j] > m) m = w[j];
        }
        double denom = 0.0;
        for (int32_t j = 0; j < L; ++j) {
            w[j] = exp(w[j] - m);
            denom += w[j];
        }
        for (int32_t d = 0; d < D; ++d) {
            double acc = 0.0;
            for (int32_t j = 0; j < L; ++j) acc += w[j] * Vc[(int64_t)j * D + d];
            o[d] = acc / denom;
        }
    }
    free(Kc);
    free(Vc);
    free(w);
    free(qh);
    return 0;
}

static void* attn_worker(void* arg) {
    attn_job* J = (attn_job*)arg;
    int64_t items = (int64_t)J->num_seqs * J->num_kv_heads;
    J->status = 0;
    for (int64_t it = J->thread_id; it < items; it += J->num_threads) {
        int rc = attend_one(J, (int32_t)(it / J->num_kv_heads), (int32_t)(it % J->num_kv_heads));
        if (rc != 0) { J->status = rc; break; }
    }
    return NULL;
}

/*
 * out[i][h][:] = sum_j softmax_j(scale * q[i][h] . K_i[j]) * V_i[j] over the
 * first context_lens[i] logical tokens of sequence i, K_i/V_i read through the
 * block table of row i.  Work is spread over num_threads threads by
 * (sequence, KV head) pair; each pair is computed by one thread in a fixed
 * order, so the result does not depend on the thread count.
 * Returns 0, -1 for an invalid table entry or length, -2 if out of memory,
 * -3 for an invalid shape.
 */
int oracle_paged_attention(double* out, const void* q, const void* k_pool, const void* v_pool,
                           int32_t dtype, int64_t num_blocks, int32_t num_kv_heads,
                           int32_t block_size, int32_t head_dim, int32_t num_q_heads,
                           const int32_t* tables, int32_t max_blocks_per_seq,
                           const int32_t* context_lens, int32_t num_seqs, double scale,
                           int32_t num_threads) {
    if (num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0 || head_dim <= 0 || block_size <= 0) return -3;
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return -3;
    if (num_threads < 1) num_threads = 1;
    attn_job* jobs = (attn_job*)calloc((size_t)num_threads, sizeof(attn_job));
    pthread_t* th = (pthread_t*)calloc((size_t)num_threads, sizeof(pthread_t));
    if (!jobs || !th) { free(jobs); free(th); return -2; }
    for (int32_t t = 0; t < num_threads; ++t) {
        attn_job* J = &jobs[t];
        J->out = out; J->q = q; J->k_pool = k_pool; J->v_pool = v_pool; J->dtype = dtype;
        J->num_blocks = num_blocks; J->num_kv_heads = num_kv_heads; J->block_size = block_size;
        J->head_dim = head_dim; J->num_q_heads = num_q_heads; J->tables = tables;
        J->max_blocks_per_seq = max_blocks_per_seq; J->context_lens = context_lens;
        J->num_seqs = num_seqs; J->scale = scale; J->num_threads = num_threads; J->thread_id = t;
    }
    int status = 0;
    if (num_threads == 1) {
        attn_worker(&jobs[0]);
        status = jobs[0].status;
    } else {
        int32_t started = 0;
        for (; started < num_threads; ++started)
            if (pthread_create(&th[started], NULL, attn_worker, &jobs[started]) != 0) break;
        for (int32_t t = 0; t < started; ++t) pthread_join(th[t], NULL);
        if (started < num_threads) status = -2;
        for (int32_t t = 0; t < started; ++t)
            if (jobs[t].status != 0) status = jobs[t].status;
    }
    free(jobs);
    free(th);
    return status;
}
