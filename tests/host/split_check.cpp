// Host-side check of the integer arithmetic the balanced decode shares with
// its fix-up (split.hpp) and of the table-entry arithmetic of the tile walks
// (table_index.hpp), built with g++ and the address / undefined-behaviour
// sanitizers.  The slice walk below restates the decode kernel's loop over
// the pieces of one worker's slice; over many random batches it checks that
// every tile of every (sequence, KV head) walk is walked exactly once, that a
// worker leaves at most its two partial records (the first piece's and the
// last one's), and that the fix-up's record lookup finds exactly the records
// each split walk left.
#include <cstdint>
#include <cstdio>
#include <cmath>
#include <algorithm>
#include <cstdlib>
#include <map>
#include <random>
#include <vector>

#include "split.hpp"
#include "table_index.hpp"

namespace {

int failures = 0;
#define CHECK(cond, ...)                                            \
    do {                                                            \
        if (!(cond)) {                                              \
            if (failures < 20) {                                    \
                std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
                std::fprintf(stderr, __VA_ARGS__);                  \
                std::fprintf(stderr, "\n");                         \
            }                                                       \
            ++failures;                                             \
        }                                                           \
    } while (0)

constexpr int kTile = 16;

struct Batch {
    std::vector<int> nblk;   // tiles per (sequence, KV head) walk
    int hkv;
};

void check_split(const Batch& bt, int64_t W, kvp::SliceWeights kw, int cost) {
    const int S = (int)bt.nblk.size(), Hkv = bt.hkv;
    std::vector<int64_t> first(S + 1, 0);
    for (int i = 0; i < S; ++i) first[i + 1] = first[i] + (int64_t)Hkv * kvp::walk_span(bt.nblk[i], cost);
    const int64_t T = first[S];
    // walked[seq][kv][b] = worker
    std::vector<std::vector<std::vector<int64_t>>> walked(S);
    for (int i = 0; i < S; ++i) walked[i].assign(Hkv, std::vector<int64_t>(bt.nblk[i], -1));
    std::map<int64_t, std::pair<int, int>> records;   // record slot -> walk
    if (T == 0) return;
    const kvp::SplitConsts sc = kvp::split_consts(W, kw);
    const double rcp_T = 1.0 / (double)T;
    for (int64_t w = 0; w < W; ++w) {
        int64_t t = kvp::slice_start(w, T, sc);
        const int64_t t_end = kvp::slice_start(w + 1, T, sc);
        CHECK(t <= t_end && t_end <= T, "slice bounds w=%lld", (long long)w);
        if (t >= t_end) continue;
        int seq = 0;
        while (!(first[seq] <= t && t < first[seq + 1])) ++seq;   // a sequence with positions
        int nblk = bt.nblk[seq];
        const int64_t span = kvp::walk_span(nblk, cost);
        const int64_t off = t - first[seq];
        int kv = (int)(off / span);
        const int64_t at = off - (int64_t)kv * span;
        int b = kvp::first_tile_at(at, cost);
        t += cost + b - at;
        bool first_piece = true;
        while (t < t_end && seq < S) {
            const int n_here = (int)std::min<int64_t>(nblk - b, t_end - t);
            CHECK(n_here >= 1 && b + n_here <= nblk, "piece w=%lld seq=%d kv=%d b=%d n=%d", (long long)w, seq, kv, b,
                  n_here);
            const bool whole = b == 0 && n_here == nblk;
            for (int k = b; k < b + n_here; ++k) {
                CHECK(walked[seq][kv][k] == -1, "tile walked twice seq=%d kv=%d b=%d", seq, kv, k);
                walked[seq][kv][k] = w;
            }
            if (!whole) {
                const int64_t slot = 2 * w + (first_piece ? 0 : 1);
                CHECK(records.count(slot) == 0, "record slot %lld written twice", (long long)slot);
                records[slot] = {seq, kv};
            }
            t += n_here;
            first_piece = false;
            b += n_here;
            if (b == nblk) {
                b = 0;
                if (++kv == Hkv) {
                    kv = 0;
                    do {
                        ++seq;
                        nblk = seq < S ? bt.nblk[seq] : 0;
                    } while (nblk == 0 && seq < S && t < t_end);
                }
                t += cost;
            }
        }
    }
    // every tile once; the fix-up's lookup
    std::map<std::pair<int, int>, int> recs_per_walk;
    for (auto& r : records) recs_per_walk[r.second]++;
    for (int seq = 0; seq < S; ++seq) {
        const int nblk = bt.nblk[seq];
        for (int kv = 0; kv < Hkv; ++kv) {
            for (int k = 0; k < nblk; ++k) CHECK(walked[seq][kv][k] >= 0, "tile not walked seq=%d kv=%d b=%d", seq, kv, k);
            if (nblk == 0) continue;
            const int64_t base = first[seq] + (int64_t)kv * kvp::walk_span(nblk, cost);
            const int64_t s0 = base + cost;
            const int64_t w0 = kvp::worker_of(s0, T, rcp_T, sc), w1 = kvp::worker_of(s0 + nblk - 1, T, rcp_T, sc);
            CHECK(walked[seq][kv][0] == w0 && walked[seq][kv][nblk - 1] == w1, "owners seq=%d kv=%d", seq, kv);
            if (w0 == w1) {
                CHECK(recs_per_walk.count(std::make_pair(seq, kv)) == 0, "whole walk left a record seq=%d kv=%d", seq, kv);
                continue;
            }
            int found = 0;
            for (int64_t w = w0; w <= w1; ++w) {
                const int64_t st = kvp::slice_start(w, T, sc);
                if (kvp::slice_start(w + 1, T, sc) <= st) continue;   // empty slice
                const int64_t slot = (w == w0 && st < base) ? 2 * w + 1 : 2 * w;
                auto it = records.find(slot);
                CHECK(it != records.end() && it->second == std::make_pair(seq, kv),
                      "fix-up looks for slot %lld of seq=%d kv=%d", (long long)slot, seq, kv);
                ++found;
            }
            const int left = recs_per_walk[std::make_pair(seq, kv)];
            CHECK(found == left, "records of seq=%d kv=%d: %d looked up, %d left", seq, kv, found, left);
        }
    }
    // worker_of inverts slice_start
    for (int64_t t = 0; t < T; t += 1 + T / 5000) {
        const int64_t w = kvp::worker_of(t, T, rcp_T, sc);
        CHECK(kvp::slice_start(w, T, sc) <= t && t < kvp::slice_start(w + 1, T, sc), "worker_of t=%lld",
              (long long)t);
    }
}

void check_table_index() {
    for (int B : {8, 16, 32, 64, 128}) {
        const bool pair8 = B == 8;
        int sub_shift = 0;
        while ((kTile << sub_shift) < B) ++sub_shift;
        if (B < kTile) sub_shift = 0;
        for (int row_len = 0; row_len <= 300; ++row_len) {
            const int tokens = row_len * B;
            const int tiles = (tokens + kTile - 1) / kTile;
            for (int e = 0; e < tiles + 4; ++e) {
                const bool in_row = kvp::tile_in_row(e, row_len, pair8, sub_shift);
                CHECK(in_row == (e < tiles), "tile_in_row B=%d row_len=%d e=%d", B, row_len, e);
                if (!in_row) continue;
                const int first = kvp::tile_first_entry(e, pair8, sub_shift);
                CHECK(first == (e * kTile) / B && first < row_len, "first entry B=%d e=%d", B, e);
                const bool second = kvp::tile_has_second_entry(e, row_len, pair8);
                // B = 8: tokens 8..15 of the tile live in entry 2e + 1, which exists iff inside the row
                CHECK(second == (pair8 && 2 * e + 1 < row_len), "second entry B=%d row_len=%d e=%d", B, row_len, e);
            }
        }
    }
}

}  // namespace

void check_div_floor() {
    std::mt19937_64 rng(7);
    for (int i = 0; i < 2000000; ++i) {
        const int64_t den = 1 + (int64_t)(rng() % ((i & 1) ? 70000 : ((int64_t)1 << 31) - 1));
        int64_t num = (int64_t)(rng() % ((int64_t)1 << (i % 3 == 0 ? 50 : 47)));
        if (i % 4 == 1) num = (num / den) * den;       // exact multiples
        if (i % 4 == 2 && num >= den) num = (num / den) * den - 1;   // just below one
        CHECK(kvp::div_floor(num, den) == num / den, "div_floor(%lld, %lld)", (long long)num, (long long)den);
    }
}

// floor division by a multiply with the reciprocal: exact over its whole
// domain (num < 2^52, den < 2^31, quotient <= 2^31 - 1), exact multiples and
// remainders of den - 1 included, against integer division
void check_div_floor_rcp() {
    std::mt19937_64 rng(11);
    const int64_t kQMax = ((int64_t)1 << 31) - 1, kNumMax = ((int64_t)1 << 52) - 1;
    for (int i = 0; i < 4000000; ++i) {
        int64_t den;
        switch (i % 4) {
            case 0: den = 1 + (int64_t)(rng() % 64); break;
            case 1: den = 1 + (int64_t)(rng() % ((int64_t)1 << 21)); break;
            case 2: den = ((int64_t)1 << 31) - 1 - (int64_t)(rng() % 1024); break;
            default: den = 1 + (int64_t)(rng() % (((int64_t)1 << 31) - 1)); break;
        }
        const int64_t qmax = std::min(kQMax, (kNumMax - (den - 1)) / den);
        int64_t q = (int64_t)(rng() % (uint64_t)(qmax + 1));
        if (i % 7 == 0) q = qmax;
        if (i % 11 == 0) q = qmax - (int64_t)(rng() % 8) < 0 ? 0 : qmax - (int64_t)(rng() % 8);
        // num / den itself at most 2^31 - 1: the largest quotient only with no remainder
        const int64_t r = (i % 3 == 0 || q == kQMax) ? 0 : (i % 3 == 1 ? den - 1 : (int64_t)(rng() % (uint64_t)den));
        const int64_t num = q * den + r;
        CHECK(num >= 0 && num <= kNumMax, "domain");
        const double rcp = 1.0 / (double)den;
        CHECK(kvp::div_floor_rcp(num, den, rcp) == q, "div_floor_rcp(%lld, %lld) = %lld, want %lld", (long long)num,
              (long long)den, (long long)kvp::div_floor_rcp(num, den, rcp), (long long)q);
    }
}

// The split at its limits: the most positions one launch takes and the most
// workers, with either pool's weights
void check_split_limits() {
    for (auto kw : {kvp::kBf16SliceWeights, kvp::kFp8SliceWeights}) {
        const int64_t W = kvp::kMaxSplitWorkers;
        const kvp::SplitConsts sc = kvp::split_consts(W, kw);
        for (int64_t T : {kvp::kMaxSplitPositions - 1, kvp::kMaxSplitPositions - 2, (int64_t)1 << 30, (int64_t)12345}) {
            const double rcp_T = 1.0 / (double)T;
            CHECK(kvp::slice_start(0, T, sc) == 0 && kvp::slice_start(W, T, sc) == T, "ends T=%lld", (long long)T);
            int64_t prev = 0;
            for (int64_t w = 1; w <= W; ++w) {
                const int64_t st = kvp::slice_start(w, T, sc);
                // exact: floor(T cum(w) / cum(W)) in 128-bit integers
                const __int128 want = (__int128)T * kvp::cum_weight(w, W, kw) / sc.cum_W;
                CHECK(st == (int64_t)want && st >= prev, "slice_start w=%lld T=%lld", (long long)w, (long long)T);
                prev = st;
            }
            for (int64_t t : {(int64_t)0, T / 3, T / 2, T - 2, T - 1}) {
                const int64_t w = kvp::worker_of(t, T, rcp_T, sc);
                CHECK(kvp::slice_start(w, T, sc) <= t && t < kvp::slice_start(w + 1, T, sc), "worker_of limits");
            }
        }
    }
}

int main() {
    check_table_index();
    check_div_floor();
    check_div_floor_rcp();
    check_split_limits();
    std::mt19937_64 rng(12345);
    // the decode's weights, plain equal slices, and lopsided parity and half
    // weights (the first or the second half heavier), so that every branch of
    // worker_of's inversion is taken with odd and even worker counts
    const kvp::SliceWeights weights[] = {kvp::kBf16SliceWeights, kvp::kFp8SliceWeights, {1, 1, 1, 1},
                                         {3, 1, 5, 2}, {1, 4, 2, 7}};
    const int64_t workers[] = {1, 7, 64, 1024, 2048, 2049};
    int cases = 0;
    for (int rep = 0; rep < 60; ++rep) {
        Batch bt;
        bt.hkv = (int)std::vector<int>{1, 2, 8}[rep % 3];
        const int S = 1 + (int)(rng() % (rep % 4 == 0 ? 300 : 64));
        std::lognormal_distribution<double> ln(std::log(64.0), 1.0);
        for (int i = 0; i < S; ++i) {
            int n;
            switch (rng() % 5) {
                case 0: n = 0; break;                       // empty sequence
                case 1: n = 1 + (int)(rng() % 3); break;    // a tile or three
                default: n = std::min(512, (int)ln(rng)); break;
            }
            bt.nblk.push_back(n);
        }
        for (auto kw : weights)
            for (int64_t W : workers)
                for (int cost : {0, 1, kvp::kBf16PieceCost, kvp::kFp8PieceCost, 7}) {
                    check_split(bt, W, kw, cost);
                    ++cases;
                }
    }
    // all-empty and single-walk batches
    check_split(Batch{{0, 0, 0}, 8}, 1024, kvp::kBf16SliceWeights, kvp::kBf16PieceCost);
    check_split(Batch{{1}, 1}, 1024, kvp::kBf16SliceWeights, kvp::kBf16PieceCost);
    check_split(Batch{{5000}, 1}, 1024, kvp::kFp8SliceWeights, kvp::kFp8PieceCost);
    std::printf("%d split cases, %s\n", cases + 3, failures ? "FAILED" : "ok");
    return failures ? 1 : 0;
}
