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
//   cum(w) = even ceil(w / 2) + odd floor(w / 2),  cum(2p) = (even + odd) p,  cum(2p + 1) = (even + odd) p + even
struct SliceWeights {
    int64_t even, odd;
};
constexpr SliceWeights kBf16SliceWeights{33, 32};
constexpr SliceWeights kFp8SliceWeights{21, 20};

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
// (and T cum(W) must stay below 2^53 for div_floor): batches with more
// positions take another kernel.
constexpr int64_t kMaxSplitPositions = (int64_t)1 << 31;

KVP_SPLIT_HD inline int64_t cum_weight(int64_t w, SliceWeights k) {
    return k.even * ((w + 1) / 2) + k.odd * (w / 2);
}
KVP_SPLIT_HD inline int64_t slice_start(int64_t w, int64_t T, int64_t W, SliceWeights k) {
    return div_floor(T * cum_weight(w, k), cum_weight(W, k));
}

// Worker whose slice holds tile t (0 <= t < T): the largest w with
// slice_start(w) <= t, i.e. cum(w) T <= (t + 1) cum(W) - 1, i.e.
// cum(w) <= X = floor(((t + 1) cum(W) - 1) / T); with X = (even + odd) p + r
// that is w = 2p + 1 when r >= even, else 2p.
KVP_SPLIT_HD inline int64_t worker_of(int64_t t, int64_t T, int64_t W, SliceWeights k) {
    const int64_t X = div_floor((t + 1) * cum_weight(W, k) - 1, T);
    const int64_t pair = k.even + k.odd;
    const int64_t p = div_floor(X, pair);
    const int64_t w = 2 * p + (X - p * pair >= k.even ? 1 : 0);
    return w < W - 1 ? w : W - 1;
}

}  // namespace kvp
