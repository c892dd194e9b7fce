// Which block-table entries a 16-token K/V tile reads.  Plain integer
// arithmetic, shared by the decode kernels and by a host-side test that
// checks it against the row bounds for every block size and row length
// (this header includes nothing from HIP, so a host compiler takes it as is).
//
// A table row lists the physical block of each B-token logical block
// ("PagedAttention, Internals First", "02 Block tables": token t lives in
// logical block t / B).  The kernels walk 16-token tiles whatever B is:
//   * B >= 16: tile e lies in logical block e / (B / 16) (sub_shift =
//     log2(B / 16));
//   * B = 8: tile e covers logical blocks 2e (tokens 0..7) and 2e + 1
//     (tokens 8..15); the second exists only while 2e + 1 is inside the row,
//     so the last tile of a row with an odd number of entries has one block.
// `row_len` is the number of entries the row pointer can address: the whole
// row, or what follows a shared prefix when the walk starts after it.
#pragma once

#if defined(__HIPCC__)
#define KVP_HOST_DEVICE __host__ __device__
#else
#define KVP_HOST_DEVICE
#endif

namespace kvp {

// Entry of the block holding tokens 0..7 (B = 8) or all 16 tokens (B >= 16) of tile e.
KVP_HOST_DEVICE inline int tile_first_entry(int e, bool pair8, int sub_shift) {
    return pair8 ? 2 * e : e >> sub_shift;
}

// Whether tile e has a second block (B = 8) inside a row of row_len entries.
KVP_HOST_DEVICE inline bool tile_has_second_entry(int e, int row_len, bool pair8) {
    return pair8 && 2 * e + 1 < row_len;
}

// Whether tile e starts inside a row of row_len entries (its first entry exists).
KVP_HOST_DEVICE inline bool tile_in_row(int e, int row_len, bool pair8, int sub_shift) {
    return tile_first_entry(e, pair8, sub_shift) < row_len;
}

}  // namespace kvp
