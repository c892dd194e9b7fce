// The C-ABI layer's host-only checks (paged_kv_cache_num_amd/csrc/host_logic.hpp)
// built with g++ under the address and undefined-behaviour sanitizers, once
// as the release library compiles them and once as the KV_DEBUG build does:
// pool and scale sizes (with 64-bit overflow), descriptor checks, and the slot
// mapping against positions written out one by one, with every error return
// and, in the debug build, the refusal of two writes to one slot.
#include <cstdint>
#include <algorithm>
#include <cstdio>
#include <random>
#include <vector>

#include "host_logic.hpp"

#ifndef CHECK_DEBUG
#define CHECK_DEBUG 0
#endif

namespace {
int failures = 0;
#define CHECK(cond, ...)                                                  \
    do {                                                                  \
        if (!(cond)) {                                                    \
            std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__);     \
            std::fprintf(stderr, __VA_ARGS__);                            \
            std::fprintf(stderr, "\n");                                   \
            ++failures;                                                   \
        }                                                                 \
    } while (0)

using kvp::host::Message;

void check_sizes() {
    Message m;
    kv_pool_desc d{2, 100, 16, 8, 128, KV_BF16};
    uint64_t b = 0;
    CHECK(kvp::host::pool_bytes(&d, &b, m) == KV_OK && b == 2ull * 100 * 16 * 8 * 128 * 2, "bf16 pool bytes %llu",
          (unsigned long long)b);
    CHECK(kvp::host::scale_bytes(&d, &b, m) == KV_OK && b == 0, "bf16 pool has no scales");
    d.dtype = KV_FP8_E4M3;
    CHECK(kvp::host::pool_bytes(&d, &b, m) == KV_OK && b == 2ull * 100 * 16 * 8 * 128, "fp8 pool bytes");
    CHECK(kvp::host::scale_bytes(&d, &b, m) == KV_OK && b == 4ull * 8 * 100 * 2, "fp8 scale bytes");
    kv_pool_desc big{1 << 30, 1 << 30, 1 << 20, 1 << 20, 1 << 20, KV_F32};
    CHECK(kvp::host::pool_bytes(&big, &b, m) == KV_ERR_INVALID_ARGUMENT, "64-bit overflow refused");
    kv_pool_desc bad{1, 0, 16, 8, 128, KV_BF16};
    CHECK(kvp::host::pool_bytes(&bad, &b, m) == KV_ERR_INVALID_ARGUMENT, "zero blocks refused");
    kv_pool_desc bad_t{1, 4, 16, 8, 128, 7};
    CHECK(kvp::host::check_desc(&bad_t, m) == KV_ERR_INVALID_ARGUMENT, "unknown dtype refused");
    CHECK(kvp::host::check_desc(nullptr, m) == KV_ERR_INVALID_ARGUMENT, "NULL descriptor refused");
}

void check_slot_mapping() {
    std::mt19937 rng(5);
    for (int rep = 0; rep < 300; ++rep) {
        const int R = 1 + (int)(rng() % 9), MB = 1 + (int)(rng() % 12), N = 1 + (int)(rng() % 200);
        const int B = 1 << (3 + (int)(rng() % 5));
        std::vector<int32_t> tables((size_t)R * MB);
        for (auto& t : tables) t = (int32_t)(rng() % N);
        const int Q = (int)(rng() % 6);
        std::vector<int32_t> seq(Q), start(Q), count(Q);
        std::vector<int64_t> want;
        for (int r = 0; r < Q; ++r) {
            seq[r] = (int32_t)(rng() % R);
            count[r] = (int32_t)(rng() % std::min(B + 3, MB * B + 1));   // a request stays inside its row
            start[r] = (int32_t)(rng() % (MB * B - count[r] + 1));
            for (int k = 0; k < count[r]; ++k) {
                const int p = start[r] + k;
                want.push_back((int64_t)tables[(size_t)seq[r] * MB + p / B] * B + p % B);
            }
        }
        std::vector<int64_t> got(want.size() + 4, -7);
        int64_t n = -1;
        Message m;
        const kv_status s = kvp::host::build_slot_mapping(tables.data(), R, MB, B, N, seq.data(), start.data(),
                                                          count.data(), Q, got.data(), (int64_t)got.size(), &n,
                                                          CHECK_DEBUG != 0, m);
        bool dup = false;
        {
            std::vector<int64_t> w = want;
            std::sort(w.begin(), w.end());
            dup = std::adjacent_find(w.begin(), w.end()) != w.end();
        }
        if (CHECK_DEBUG && dup) {
            CHECK(s == KV_ERR_INVALID_ARGUMENT && n == 0, "debug build must refuse a slot written twice");
            continue;
        }
        CHECK(s == KV_OK && n == (int64_t)want.size(), "status %d, %lld slots for %zu", (int)s, (long long)n, want.size());
        for (size_t i = 0; i < want.size() && s == KV_OK; ++i) CHECK(got[i] == want[i], "slot %zu", i);
        if (!want.empty()) {   // one entry short: refused, nothing past the end written
            std::vector<int64_t> small(want.size() - 1 + 1, -7);
            const kv_status s2 = kvp::host::build_slot_mapping(tables.data(), R, MB, B, N, seq.data(), start.data(),
                                                               count.data(), Q, small.data(), (int64_t)want.size() - 1,
                                                               &n, CHECK_DEBUG != 0, m);
            CHECK(s2 == KV_ERR_INVALID_ARGUMENT && n == 0 && small.back() == -7, "capacity one short");
        }
    }
    // error returns
    int32_t table[4] = {0, 1, 2, 9};   // entry 3 is outside a 9-block pool
    int32_t seq[1] = {0}, start[1] = {48}, count[1] = {1};
    int64_t slots[8], n = 0;
    Message m;
    CHECK(kvp::host::build_slot_mapping(table, 1, 4, 16, 9, seq, start, count, 1, slots, 8, &n, false, m) ==
              KV_ERR_OUT_OF_RANGE, "entry outside the pool");
    start[0] = 64;
    CHECK(kvp::host::build_slot_mapping(table, 1, 4, 16, 9, seq, start, count, 1, slots, 8, &n, false, m) ==
              KV_ERR_OUT_OF_RANGE, "position past the row");
    seq[0] = 1;
    start[0] = 0;
    CHECK(kvp::host::build_slot_mapping(table, 1, 4, 16, 9, seq, start, count, 1, slots, 8, &n, false, m) ==
              KV_ERR_INVALID_ARGUMENT, "row outside the table");
    seq[0] = 0;
    count[0] = -1;
    CHECK(kvp::host::build_slot_mapping(table, 1, 4, 16, 9, seq, start, count, 1, slots, 8, &n, false, m) ==
              KV_ERR_INVALID_ARGUMENT, "negative count");
    CHECK(kvp::host::build_slot_mapping(table, 1, 4, 16, 9, seq, start, count, 1, slots, 8, nullptr, false, m) ==
              KV_ERR_INVALID_ARGUMENT, "NULL num_tokens");
    // two requests writing one position: accepted by the release checks, refused by the debug ones
    int32_t seq2[2] = {0, 0}, start2[2] = {5, 5}, count2[2] = {1, 1};
    const kv_status s = kvp::host::build_slot_mapping(table, 1, 4, 16, 9, seq2, start2, count2, 2, slots, 8, &n,
                                                      CHECK_DEBUG != 0, m);
    CHECK(CHECK_DEBUG ? (s == KV_ERR_INVALID_ARGUMENT && n == 0) : (s == KV_OK && n == 2), "duplicate slot, debug=%d",
          CHECK_DEBUG);
}
}  // namespace

int main() {
    check_sizes();
    check_slot_mapping();
    std::printf("host checks (debug=%d) %s\n", CHECK_DEBUG, failures ? "FAILED" : "ok");
    return failures ? 1 : 0;
}
