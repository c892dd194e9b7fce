// Balanced split of the flattened (sequence, KV head, block) tile list into
// one contiguous slice per worker wave; shared by the decode kernel and the
// table-walk probe, so the probe walks exactly the decode's slices.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvp {

// Slice sizes.  Workgroups are dispatched round-robin over the eight XCDs,
// so worker w runs on XCD w % 8.  Measured on MI355X (per-worker exit times
// from the chip's realtime counter, and the XCC_ID register), the
// odd-numbered XCDs stream the same tiles about 6 % slower than their even
// neighbours, with the attention math or without it; a worker on an odd XCD
// therefore gets 15 tiles for every 16 of a worker on an even one.  The
// boundaries stay a function of T and W alone.
//   cum(w) = 16 ceil(w / 2) + 15 floor(w / 2),  cum(2p) = 31p,  cum(2p + 1) = 31p + 16
constexpr int64_t kEvenWeight = 16;
constexpr int64_t kOddWeight = 15;
__host__ __device__ inline int64_t cum_weight(int64_t w) {
    return kEvenWeight * ((w + 1) / 2) + kOddWeight * (w / 2);
}
__host__ __device__ inline int64_t slice_start(int64_t w, int64_t T, int64_t W) {
    return T * cum_weight(w) / cum_weight(W);
}

// Worker whose slice holds tile t (0 <= t < T): the largest w with
// slice_start(w) <= t, i.e. cum(w) T <= (t + 1) cum(W) - 1, i.e.
// cum(w) <= X = floor(((t + 1) cum(W) - 1) / T); with X = 31p + r that is
// w = 2p + 1 when r >= 16, else 2p.
__host__ __device__ inline int64_t worker_of(int64_t t, int64_t T, int64_t W) {
    const int64_t X = ((t + 1) * cum_weight(W) - 1) / T;
    const int64_t pair = kEvenWeight + kOddWeight;
    const int64_t w = 2 * (X / pair) + (X % pair >= kEvenWeight ? 1 : 0);
    return w < W - 1 ? w : W - 1;
}

}  // namespace kvp
