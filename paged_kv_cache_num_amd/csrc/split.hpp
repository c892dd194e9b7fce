// Balanced split of the flattened (sequence, KV head, block) tile list into
// one contiguous slice per worker wave; shared by the decode kernel and the
// table-walk probe, so the probe walks exactly the decode's slices.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#include <hip/hip_runtime.h>
#define KVP_SPLIT_HD __host__ __device__
#else
#define KVP_SPLIT_HD
#endif

namespace kvp {

// Split positions.  A (sequence, KV head) walk of nblk tiles takes nblk +
// cost positions of the list that is cut into slices: `cost` positions before
// its tiles stand for what starting a walk costs a worker (query, table
// entries and the first tiles in flight before anything streams).  Measured
// per worker on the 70B-shaped batch with the chip's realtime counter, a walk
// start costs about one tile's time, and the workers that fell on runs of
// short sequences (ten to sixteen walks each) finished 15-30 us after the
// others.  Timed end to end (warm calls, layer after layer), bf16 tiles do
// best with 2 (70B shape 294 -> 284 us, its TP-8 shard 57.6 -> 55.8 us), FP8
// tiles, which stream twice as fast, with 3 (70B shape 189 -> 179 us); the
// 8B shape moves by under 1 us.  Tile k of the walk sits at position cost + k
// of its span; a slice that starts among the leading positions starts the
// walk at tile 0, and one that ends there leaves the walk to the next worker.
// A walk with no tiles takes no positions.
constexpr int kBf16PieceCost = 2;
constexpr int kFp8PieceCost = 3;
KVP_SPLIT_HD inline int64_t walk_span(int nblk, int cost) { return nblk > 0 ? (int64_t)nblk + cost : 0; }
// The first tile a slice starting at position `off` of a walk's span walks.
KVP_SPLIT_HD inline int first_tile_at(int64_t off, int cost) { return off > cost ? (int)(off - cost) : 0; }

// Slice sizes.  Workgroups are dispatched round-robin over the eight XCDs,
// so worker w runs on XCD w % 8.  Measured on MI355X (per-worker exit times
// from the chip's realtime counter, and the XCC_ID register), the
// odd-numbered XCDs stream the same tiles a few percent slower than their even
// neighbours, with the attention math or without it: over repeated calls of
// the 8B- and 70B-shaped batches, layer after layer, 2.8-3.2% for bf16 tiles
// and 4.9% for FP8 tiles.  A worker on an even XCD therefore gets `even`
// tiles for every `odd` of a worker on an odd one; the boundaries stay a
// function of T, W and the weights alone.
//   C(w) = even ceil(w / 2) + odd floor(w / 2),  C(2p) = (even + odd) p,  C(2p + 1) = (even + odd) p + even
// With two worker waves on every SIMD (FP8 tiles), the second half of the
// workers is dispatched after the first has taken a wave slot on every SIMD,
// and the older wave on a SIMD wins its issue arbitration: on the 8B-shaped
// batch the workers past W/2 ended 2.2% later than the others, in one clean
// step at W/2.  The first half's weights are multiplied by `lead`, the second
// half's by `trail`:
//   cum(w) = lead C(min(w, W/2)) + trail (C(w) - C(min(w, W/2)))
constexpr int64_t kFp8Lead = 45, kFp8Trail = 44;
struct SliceWeights {
    int64_t even, odd;
    int64_t lead, trail;
};
constexpr SliceWeights kBf16SliceWeights{33, 32, 1, 1};
constexpr SliceWeights kFp8SliceWeights{21, 20, kFp8Lead, kFp8Trail};

// floor(num / den) for 0 <= num < 2^53 and 0 < den < 2^31.  The quotient in
// double precision is within one of the answer (both operands are exact and
// the division is correctly rounded), so one step each way makes it exact; on
// the GPU this takes a few dozen instructions where a 64-bit integer division
// is a long software sequence.
KVP_SPLIT_HD inline int64_t div_floor(int64_t num, int64_t den) {
    int64_t q = (int64_t)((double)num / (double)den);
    if (q * den > num) {
        --q;
    } else if ((q + 1) * den <= num) {
        ++q;
    }
    return q;
}

// The balanced split's positions are counted in 32 bits in the kernel's scan
// (and T cum(W) must stay below 2^53 for the divisions): batches with more
// positions take another kernel, and the worker count is capped so that
// cum(W) <= max(lead, trail) max(even, odd) W stays below 2^21.
constexpr int64_t kMaxSplitPositions = (int64_t)1 << 31;
constexpr int kMaxSplitWorkers = 2048;
static_assert(kMaxSplitPositions * (kFp8SliceWeights.lead * kFp8SliceWeights.even * kMaxSplitWorkers) <
                      ((int64_t)1 << 53) &&
                  kMaxSplitPositions * (kBf16SliceWeights.lead * kBf16SliceWeights.even * kMaxSplitWorkers) <
                      ((int64_t)1 << 53),
              "split positions times cum(W) must stay exact in double precision");

// floor(num / den) given rcp, the double nearest 1 / den, for integers held
// exactly in doubles with 0 <= num < 2^52, 0 < den < 2^31 and num / den <=
// 2^31 - 1: num * rcp is within (num / den) 2^-52 (< 2^-21) of num / den, so
// it stays below 2^31 and its truncation is off by at most one, which one step
// corrects; the step's products stay below 2^53, so they and its comparisons
// are exact.  Multiplies where a division and 64-bit integer products would
// be: a double division is a chain of a dozen dependent instructions on the
// GPU and a 64-bit product several quarter-rate ones, and this arithmetic sits
// on the path of every worker's start and of the fix-up (its two worker_of
// calls took about 1 us of a call with divisions).
KVP_SPLIT_HD inline int64_t div_floor_rcp_d(double num, double den, double rcp) {
    int64_t q = (int64_t)(int32_t)(num * rcp);
    if ((double)q * den > num) {
        --q;
    } else if ((double)(q + 1) * den <= num) {
        ++q;
    }
    return q;
}
KVP_SPLIT_HD inline int64_t div_floor_rcp(int64_t num, int64_t den, double rcp) {
    return div_floor_rcp_d((double)num, (double)den, rcp);
}

// C(w) and cum(w) for 0 <= w <= W <= kMaxSplitWorkers (and the host check's
// odd weights and counts): every product and sum stays far below 2^31.
KVP_SPLIT_HD inline int64_t parity_weight(int64_t w, SliceWeights k) {
    const int32_t v = (int32_t)w;
    return (int64_t)((int32_t)k.even * ((v + 1) >> 1) + (int32_t)k.odd * (v >> 1));
}
KVP_SPLIT_HD inline int64_t cum_weight(int64_t w, int64_t W, SliceWeights k) {
    const int32_t ch = (int32_t)parity_weight(w < W / 2 ? w : W / 2, k);
    return (int64_t)((int32_t)k.lead * ch + (int32_t)k.trail * ((int32_t)parity_weight(w, k) - ch));
}

// One launch's split: W workers, the weights, cum(W), and the reciprocals of
// the divisors that do not depend on the batch (set on the host, so a kernel
// divides only by T, once).
struct SplitConsts {
    SliceWeights k;
    int64_t W, cum_W;
    double rcp_cum_W, rcp_pair, rcp_lead, rcp_trail;
};
KVP_SPLIT_HD inline SplitConsts split_consts(int64_t W, SliceWeights k) {
    SplitConsts s;
    s.k = k;
    s.W = W;
    s.cum_W = cum_weight(W, W, k);
    s.rcp_cum_W = 1.0 / (double)s.cum_W;
    s.rcp_pair = 1.0 / (double)(k.even + k.odd);
    s.rcp_lead = 1.0 / (double)k.lead;
    s.rcp_trail = 1.0 / (double)k.trail;
    return s;
}

// the largest w with C(w) <= Y: with Y = (even + odd) p + r, w = 2p + 1 when r >= even, else 2p
KVP_SPLIT_HD inline int64_t parity_inverse(int64_t Y, const SplitConsts& s) {
    const int64_t pair = s.k.even + s.k.odd;
    const int64_t p = div_floor_rcp(Y, pair, s.rcp_pair);
    return 2 * p + (Y - p * pair >= s.k.even ? 1 : 0);
}
// T cum(w) < 2^52 (T < kMaxSplitPositions, cum(W) < 2^21) is exact as a
// double product; the quotient is at most T < 2^31
KVP_SPLIT_HD inline int64_t slice_start(int64_t w, int64_t T, const SplitConsts& s) {
    return div_floor_rcp_d((double)T * (double)cum_weight(w, s.W, s.k), (double)s.cum_W, s.rcp_cum_W);
}

// Worker whose slice holds tile t (0 <= t < T; rcp_T the double nearest
// 1 / T): the largest w with slice_start(w) <= t, i.e. cum(w) T <= (t + 1)
// cum(W) - 1, i.e. cum(w) <= X = floor(((t + 1) cum(W) - 1) / T) (X < cum(W)).
// Below the first half's total lead C(W/2) that is C(w) <= floor(X / lead);
// above it C(w) <= C(W/2) + floor((X - lead C(W/2)) / trail).
KVP_SPLIT_HD inline int64_t worker_of(int64_t t, int64_t T, double rcp_T, const SplitConsts& s) {
    const int64_t X = div_floor_rcp_d((double)(t + 1) * (double)s.cum_W - 1.0, (double)T, rcp_T);
    const int64_t ch = parity_weight(s.W / 2, s.k);
    const int64_t w = X < s.k.lead * ch ? parity_inverse(div_floor_rcp(X, s.k.lead, s.rcp_lead), s)
                                        : parity_inverse(ch + div_floor_rcp(X - s.k.lead * ch, s.k.trail, s.rcp_trail), s);
    return w < s.W - 1 ? w : s.W - 1;
}

}  // namespace kvp
