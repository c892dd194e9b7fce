/*
 * The CPU oracle (oracle/oracle.c) built with gcc under the address and
 * undefined-behaviour sanitizers and run on small cases: slot mapping
 * against the table arithmetic written out per position, scatter as a row
 * copy that leaves every other byte alone, attention on cases with a closed
 * form (one token: the value row; equal keys: the mean of the values; an
 * empty context: zeros), thread counts that must not change a bit, and the
 * error returns for a table entry outside the pool, a request past its row
 * and a slot past the pool.  Test infrastructure only, like the oracle.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int64_t oracle_slot_mapping(const int32_t* tables, int32_t num_rows, int32_t max_blocks_per_seq,
                            int32_t block_size, int64_t num_blocks, const int32_t* write_seq,
                            const int32_t* write_start, const int32_t* write_count, int32_t num_requests,
                            int64_t* slots, int64_t capacity);
int oracle_scatter(uint8_t* k_pool, uint8_t* v_pool, int64_t num_blocks, int32_t num_kv_heads, int32_t block_size,
                   int32_t head_dim, int32_t elem_bytes, const uint8_t* k_new, const uint8_t* v_new,
                   const int64_t* slot_mapping, int64_t num_tokens);
int oracle_paged_attention(double* out, const void* q, const void* k_pool, const void* v_pool, int32_t dtype,
                           int64_t num_blocks, int32_t num_kv_heads, int32_t block_size, int32_t head_dim,
                           int32_t num_q_heads, const int32_t* tables, int32_t max_blocks_per_seq,
                           const int32_t* context_lens, int32_t num_seqs, double scale, int32_t num_threads);

static int failures = 0;
#define CHECK(c, ...)                                        \
    do {                                                     \
        if (!(c)) {                                          \
            fprintf(stderr, "FAIL line %d: ", __LINE__);     \
            fprintf(stderr, __VA_ARGS__);                    \
            fprintf(stderr, "\n");                           \
            ++failures;                                      \
        }                                                    \
    } while (0)

static uint64_t rng_state = 88172645463325252ull;
static uint64_t rnd(void) {   /* xorshift64 */
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return rng_state;
}

static void check_slot_mapping(void) {
    enum { R = 5, MB = 6, B = 8, N = 40 };
    int32_t tables[R * MB];
    for (int i = 0; i < R * MB; ++i) tables[i] = (int32_t)(rnd() % N);
    int32_t seq[] = {0, 3, 4, 1}, start[] = {0, 13, 47, 5}, count[] = {9, 20, 1, 0};
    int64_t slots[64];
    int64_t n = oracle_slot_mapping(tables, R, MB, B, N, seq, start, count, 4, slots, 64);
    CHECK(n == 30, "slot count %lld", (long long)n);
    int64_t t = 0;
    for (int r = 0; r < 4; ++r)
        for (int k = 0; k < count[r]; ++k, ++t) {
            int p = start[r] + k;
            CHECK(slots[t] == (int64_t)tables[seq[r] * MB + p / B] * B + p % B, "slot %lld", (long long)t);
        }
    int32_t past[] = {48};   /* position 48 needs entry 6 of a 6-entry row */
    int32_t one[] = {1};
    CHECK(oracle_slot_mapping(tables, R, MB, B, N, seq, past, one, 1, slots, 64) == -1, "past the row");
    tables[0] = N;           /* entry outside the pool */
    int32_t zero[] = {0};
    CHECK(oracle_slot_mapping(tables, R, MB, B, N, zero, zero, one, 1, slots, 64) == -1, "entry outside the pool");
    int32_t bad_row[] = {R};
    CHECK(oracle_slot_mapping(tables, R, MB, B, N, bad_row, zero, one, 1, slots, 64) == -1, "row outside the table");
    CHECK(oracle_slot_mapping(tables, R, MB, B, N, seq, start, count, 4, slots, 3) == -1, "capacity");
}

static void check_scatter(void) {
    enum { N = 7, H = 3, B = 4, D = 16, E = 2, T = 5 };
    const size_t pool = (size_t)N * H * B * D * E, rows = (size_t)T * H * D * E;
    uint8_t *kp = malloc(pool), *vp = malloc(pool), *k0 = malloc(pool), *v0 = malloc(pool);
    uint8_t *kn = malloc(rows), *vn = malloc(rows);
    for (size_t i = 0; i < pool; ++i) { kp[i] = (uint8_t)rnd(); vp[i] = (uint8_t)rnd(); }
    for (size_t i = 0; i < rows; ++i) { kn[i] = (uint8_t)rnd(); vn[i] = (uint8_t)rnd(); }
    memcpy(k0, kp, pool);
    memcpy(v0, vp, pool);
    int64_t slots[T] = {22, -1, 0, 13, (int64_t)N * B - 1};
    CHECK(oracle_scatter(kp, vp, N, H, B, D, E, kn, vn, slots, T) == 0, "scatter status");
    for (int t = 0; t < T; ++t) {
        if (slots[t] < 0) continue;
        int64_t blk = slots[t] / B, off = slots[t] % B;
        for (int h = 0; h < H; ++h) {
            size_t dst = (size_t)(((blk * H + h) * B + off) * D * E), src = (size_t)((t * H + h) * D * E);
            CHECK(memcmp(kp + dst, kn + src, D * E) == 0 && memcmp(vp + dst, vn + src, D * E) == 0, "row t=%d h=%d", t, h);
            memcpy(kp + dst, k0 + dst, D * E);   /* put the old bytes back: the rest must be untouched */
            memcpy(vp + dst, v0 + dst, D * E);
        }
    }
    CHECK(memcmp(kp, k0, pool) == 0 && memcmp(vp, v0, pool) == 0, "bytes outside the written rows changed");
    int64_t bad[1] = {(int64_t)N * B};
    CHECK(oracle_scatter(kp, vp, N, H, B, D, E, kn, vn, bad, 1) == -1, "slot past the pool");
    free(kp); free(vp); free(k0); free(v0); free(kn); free(vn);
}

static uint16_t f32_to_bf16_trunc(float x) {
    uint32_t u;
    memcpy(&u, &x, 4);
    return (uint16_t)(u >> 16);
}

static void check_attention(void) {
    enum { S = 4, HQ = 4, HKV = 2, D = 8, B = 4, MB = 5, N = 24 };
    float *kp = malloc(sizeof(float) * N * HKV * B * D), *vp = malloc(sizeof(float) * N * HKV * B * D);
    float q[S * HQ * D];
    for (int i = 0; i < N * HKV * B * D; ++i) { kp[i] = (float)((int)(rnd() % 17) - 8) / 8.0f; vp[i] = (float)((int)(rnd() % 33) - 16) / 4.0f; }
    for (int i = 0; i < S * HQ * D; ++i) q[i] = (float)((int)(rnd() % 9) - 4) / 4.0f;
    int32_t tables[S * MB];
    for (int i = 0; i < S * MB; ++i) tables[i] = (int32_t)((i * 7 + 3) % N);
    int32_t lens[S] = {1, 0, 17, 20};
    double out1[S * HQ * D], out4[S * HQ * D];
    CHECK(oracle_paged_attention(out1, q, kp, vp, 0, N, HKV, B, D, HQ, tables, MB, lens, S, 0.35, 1) == 0, "attention status");
    CHECK(oracle_paged_attention(out4, q, kp, vp, 0, N, HKV, B, D, HQ, tables, MB, lens, S, 0.35, 4) == 0, "attention status, 4 threads");
    CHECK(memcmp(out1, out4, sizeof out1) == 0, "thread count changed the result");
    /* one token: the value row of its KV head; an empty context: zeros */
    for (int h = 0; h < HQ; ++h)
        for (int d = 0; d < D; ++d) {
            int kv = h / (HQ / HKV);
            double v = vp[((tables[0] * HKV + kv) * B + 0) * D + d];
            CHECK(out1[(0 * HQ + h) * D + d] == v, "single token h=%d d=%d", h, d);
            CHECK(out1[(1 * HQ + h) * D + d] == 0.0, "empty context h=%d d=%d", h, d);
        }
    /* sequence 2 with every key equal: the mean of its values */
    for (int p = 0; p < lens[2]; ++p)
        for (int kv = 0; kv < HKV; ++kv)
            for (int d = 0; d < D; ++d) kp[((tables[2 * MB + p / B] * HKV + kv) * B + p % B) * D + d] = 0.5f;
    CHECK(oracle_paged_attention(out1, q, kp, vp, 0, N, HKV, B, D, HQ, tables, MB, lens, S, 0.35, 2) == 0, "status");
    for (int h = 0; h < HQ; ++h)
        for (int d = 0; d < D; ++d) {
            int kv = h / (HQ / HKV);
            double mean = 0.0;
            for (int p = 0; p < lens[2]; ++p) mean += vp[((tables[2 * MB + p / B] * HKV + kv) * B + p % B) * D + d];
            mean /= lens[2];
            CHECK(fabs(out1[(2 * HQ + h) * D + d] - mean) <= 1e-12 * (1.0 + fabs(mean)), "equal keys h=%d d=%d", h, d);
        }
    /* bf16 storage: the same values truncated to bf16 give the f32 result of the truncated values */
    uint16_t *kb = malloc(2 * N * HKV * B * D), *vb = malloc(2 * N * HKV * B * D);
    uint16_t qb[S * HQ * D];
    float *kt = malloc(sizeof(float) * N * HKV * B * D), *vt = malloc(sizeof(float) * N * HKV * B * D);
    float qt[S * HQ * D];
    for (int i = 0; i < N * HKV * B * D; ++i) {
        kb[i] = f32_to_bf16_trunc(kp[i] * 1.37f); vb[i] = f32_to_bf16_trunc(vp[i] * 0.71f);
        uint32_t u = (uint32_t)kb[i] << 16; memcpy(&kt[i], &u, 4);
        u = (uint32_t)vb[i] << 16; memcpy(&vt[i], &u, 4);
    }
    for (int i = 0; i < S * HQ * D; ++i) { qb[i] = f32_to_bf16_trunc(q[i] * 1.1f); uint32_t u = (uint32_t)qb[i] << 16; memcpy(&qt[i], &u, 4); }
    CHECK(oracle_paged_attention(out1, qb, kb, vb, 1, N, HKV, B, D, HQ, tables, MB, lens, S, 0.35, 3) == 0, "bf16 status");
    CHECK(oracle_paged_attention(out4, qt, kt, vt, 0, N, HKV, B, D, HQ, tables, MB, lens, S, 0.35, 1) == 0, "f32 status");
    CHECK(memcmp(out1, out4, sizeof out1) == 0, "bf16 storage differs from the widened f32 values");
    /* error returns */
    tables[3 * MB] = N;
    CHECK(oracle_paged_attention(out1, q, kp, vp, 0, N, HKV, B, D, HQ, tables, MB, lens, S, 0.35, 2) == -1, "entry outside the pool");
    tables[3 * MB] = 0;
    lens[0] = MB * B + 1;
    CHECK(oracle_paged_attention(out1, q, kp, vp, 0, N, HKV, B, D, HQ, tables, MB, lens, S, 0.35, 1) == -1, "length past the row");
    CHECK(oracle_paged_attention(out1, q, kp, vp, 0, N, 3, B, D, HQ, tables, MB, lens, S, 0.35, 1) == -3, "group shape");
    free(kp); free(vp); free(kb); free(vb); free(kt); free(vt);
}

int main(void) {
    check_slot_mapping();
    check_scatter();
    check_attention();
    printf("oracle checks %s\n", failures ? "FAILED" : "ok");
    return failures ? 1 : 0;
}
