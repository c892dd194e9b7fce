// FP8 pools: storing rows through a slot mapping with the block scale rule,
// as device helpers for the scatter kernels and for extra waves of the decode
// step's launch.
//
// "PagedAttention, Internals First", "06 Open questions": a block is a natural
// quantization group.  The rule: the write that puts row 0 of a block in place
// sets the block's K and V scales (one per KV head) to amax / 448 over every
// row that write puts into the block; every other row is quantized with the
// scale already stored.  Slots are unique (the scatter's precondition), so a
// block has at most B writers; when tokens t .. t+B-1 hold its slots
// B*blk .. B*blk+B-1 in order no other token can write it, and that common
// case needs no search of the mapping.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.hpp"
#include "fp8.hpp"

namespace kvp {

constexpr int kFp8RowGroup = 16;      // block rows gathered per round (all of them for 8-token blocks)
constexpr int kFp8SearchUnroll = 8;   // slots per lane and step of a search of the mapping
constexpr int kFp8RowWords = 64;      // 32-bit words (bf16 pairs) per 128-dim row

__device__ __forceinline__ int64_t fp8_readlane64(int64_t x, int src) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, src);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)x >> 32), src);
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Lane i < R: the token that writes slot lo + i, or -1 when none does.  The
// run that would hold them (tokens t_run .. t_run + R - 1) is checked first;
// otherwise the whole mapping is searched, 64 * kFp8SearchUnroll slots a step.
__device__ __forceinline__ int64_t fp8_row_writers(const int64_t* __restrict__ slots, int64_t T, int64_t t_run,
                                                   int64_t lo, int R, int lane) {
    const uint64_t run_mask = R >= 64 ? ~0ull : ((1ull << R) - 1);
    const int64_t tl = t_run + lane;
    const bool in_run = lane < R && tl >= 0 && tl < T && slots[tl] == lo + lane;
    if (__builtin_amdgcn_ballot_w64(in_run) == run_mask) return in_run ? tl : -1;
    int64_t tok = -1;
    for (int64_t s0 = 0; s0 < T; s0 += kFp8SearchUnroll * kWave) {
        int64_t sl[kFp8SearchUnroll];
#pragma unroll
        for (int u = 0; u < kFp8SearchUnroll; ++u) {
            const int64_t ts = s0 + u * kWave + lane;
            sl[u] = ts < T ? slots[ts] : -1;
        }
#pragma unroll
        for (int u = 0; u < kFp8SearchUnroll; ++u) {
            uint64_t hit = __builtin_amdgcn_ballot_w64(sl[u] >= lo && sl[u] < lo + R);
            while (hit) {
                const int jj = __builtin_ctzll(hit);
                hit &= hit - 1;
                const int row = (int)(fp8_readlane64(sl[u], jj) - lo);
                if (lane == row) tok = s0 + u * kWave + jj;
            }
        }
    }
    return tok;
}

// x of lane src (0 <= src < 64)
__device__ __forceinline__ int64_t fp8_shfl64(int64_t x, int src) {
    const int lo = __shfl((int)(uint32_t)x, src, kWave);
    const int hi = __shfl((int)(uint32_t)((uint64_t)x >> 32), src, kWave);
    return (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

// Rows to store: row t (bf16, [T][H][128]) goes to `slots[t]` of an FP8 pool
// layer (codes [N][H][B][128], scales [N][H]); slots outside [0, num_slots)
// are skipped.
struct Fp8Rows {
    const int64_t* slots;
    int64_t T;
    const uint32_t* k_new;
    const uint32_t* v_new;
    uint16_t* k_codes;
    uint16_t* v_codes;
    float* k_scale;
    float* v_scale;
    int B, H;
    int64_t num_slots;
};

// One quantized row: lane l writes dims 2l and 2l + 1 of KV head h.
__device__ __forceinline__ void fp8_put_row(const Fp8Rows& r, int64_t blk, int h, int row, uint32_t kw, uint32_t vw,
                                            float ks, float vs, int lane) {
    const int64_t at = ((blk * r.H + h) * r.B + row) * kFp8RowWords + lane;
    r.k_codes[at] = (uint16_t)bf16x2_to_e4m3x2(kw, ks);
    r.v_codes[at] = (uint16_t)bf16x2_to_e4m3x2(vw, vs);
}

// Tokens c0 .. c0 + 15 of the mapping, KV head h, stored by one wave, bitwise
// as the two scatter kernels store them (fp8_scale_kernel, then
// fp8_quantize_kernel): a token writing row 0 of a block gathers the block's
// writers (kFp8RowGroup rows a round), takes the amax of their K and V rows,
// sets the block's scales and stores those rows' codes (B > 16: the rows are
// loaded again for the codes once the amax is known); a token writing any
// other row is stored here only when no token writes its block's row 0, with
// the stored scale.  Every row is thus stored once, by the wave that holds
// its block's row 0 or by its own.  A chunk of a prefill run takes three
// memory round trips: its slots, the run check of its opener (the other
// tokens find their block's row-0 token among the chunk's slots), its rows.
__device__ __forceinline__ void fp8_store_chunk(const Fp8Rows& r, int64_t c0, int h, int lane) {
    const int B = r.B;   // a power of two (8 .. 128): slots split with shifts, not 64-bit divisions
    const int bshift = __builtin_ctz((unsigned)B);
    const int R = B < kFp8RowGroup ? B : kFp8RowGroup;
    const int64_t t = c0 + lane;
    const int64_t slot = (lane < 16 && t < r.T) ? r.slots[t] : -1;
    const bool valid = slot >= 0 && slot < r.num_slots;
    const size_t hrow = (size_t)h * kFp8RowWords + lane;   // lane's word of head h in a [H][128] row
    const size_t row_words = (size_t)r.H * kFp8RowWords;

    // blocks opened by a token of this chunk
    uint64_t starts = __builtin_amdgcn_ballot_w64(valid && (slot & (B - 1)) == 0);
    while (starts) {
        const int j = __builtin_ctzll(starts);
        starts &= starts - 1;
        const int64_t first = fp8_readlane64(slot, j);
        const int64_t blk = first >> bshift;
        float ak = 0.0f, av = 0.0f;
        uint32_t wk[kFp8RowGroup], wv[kFp8RowGroup];
        int64_t tok = -1;
        for (int g = 0; g < B; g += R) {
            tok = fp8_row_writers(r.slots, r.T, c0 + j + g, first + g, R, lane);
#pragma unroll
            for (int i = 0; i < kFp8RowGroup; ++i) {
                const int64_t ti = fp8_readlane64(tok, i);
                const size_t w = (size_t)(ti < 0 ? 0 : ti) * row_words + hrow;
                wk[i] = r.k_new[w];
                wv[i] = r.v_new[w];
            }
#pragma unroll
            for (int i = 0; i < kFp8RowGroup; ++i) {
                if (i < R && fp8_readlane64(tok, i) >= 0) {
                    ak = abs_max2(wk[i], ak);
                    av = abs_max2(wv[i], av);
                }
            }
        }
        const float ks = e4m3_block_scale(wave_max(ak));
        const float vs = e4m3_block_scale(wave_max(av));
        if (lane == 0) {
            r.k_scale[blk * r.H + h] = ks;
            r.v_scale[blk * r.H + h] = vs;
        }
        for (int g = 0; g < B; g += R) {
            if (B > R) {   // the last round's rows are still in registers only when there was one round
                tok = fp8_row_writers(r.slots, r.T, c0 + j + g, first + g, R, lane);
#pragma unroll
                for (int i = 0; i < kFp8RowGroup; ++i) {
                    const int64_t ti = fp8_readlane64(tok, i);
                    const size_t w = (size_t)(ti < 0 ? 0 : ti) * row_words + hrow;
                    wk[i] = r.k_new[w];
                    wv[i] = r.v_new[w];
                }
            }
#pragma unroll
            for (int i = 0; i < kFp8RowGroup; ++i)
                if (i < R && fp8_readlane64(tok, i) >= 0) fp8_put_row(r, blk, h, g + i, wk[i], wv[i], ks, vs, lane);
        }
    }

    // The other tokens of the chunk (lanes < 16), all at once: a token is
    // stored here, with the stored scale, only when no token writes its
    // block's row 0.  The token that would (c0 + lane - offset, if the rows
    // came as a run) is checked first, from a lane of this chunk or by one
    // load; the tokens still in doubt search the mapping together.
    const bool other = valid && (slot & (B - 1)) != 0;
    const int64_t blk = other ? slot >> bshift : 0;
    const int off = other ? (int)(slot & (B - 1)) : 0;
    const int64_t want = blk << bshift;
    const int64_t tg = c0 + lane - off;
    const int src = (int)(tg - c0);   // < 16 for the tokens of this chunk
    const int64_t s_in = fp8_shfl64(slot, src >= 0 ? src : 0);
    const int64_t s_tg = src >= 0 ? s_in : ((other && tg >= 0) ? r.slots[tg] : -1);
    bool opened = other && s_tg == want;
    const uint64_t unsure = __builtin_amdgcn_ballot_w64(other && !opened);
    if (unsure) {
        uint64_t found = 0;
        for (int64_t s0 = 0; s0 < r.T; s0 += kFp8SearchUnroll * kWave) {
            int64_t sl[kFp8SearchUnroll];
#pragma unroll
            for (int u = 0; u < kFp8SearchUnroll; ++u) {
                const int64_t ts = s0 + u * kWave + lane;
                sl[u] = ts < r.T ? r.slots[ts] : -1;
            }
            uint64_t left = unsure & ~found;
            while (left) {
                const int p = __builtin_ctzll(left);
                left &= left - 1;
                const int64_t target = fp8_readlane64(want, p);
                bool hit = false;
#pragma unroll
                for (int u = 0; u < kFp8SearchUnroll; ++u) hit |= sl[u] == target;
                if (__builtin_amdgcn_ballot_w64(hit)) found |= 1ull << p;
            }
            if ((unsure & ~found) == 0) break;
        }
        opened = opened || ((found >> lane) & 1);
    }
    const uint64_t todo = __builtin_amdgcn_ballot_w64(other && !opened);
    if (todo) {
        float ks_l = 0.0f, vs_l = 0.0f;   // lane i: the stored scales of token c0 + i's block
        if ((todo >> lane) & 1) {
            ks_l = r.k_scale[blk * r.H + h];
            vs_l = r.v_scale[blk * r.H + h];
        }
        uint32_t wk[16], wv[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int64_t ti = c0 + i < r.T ? c0 + i : r.T - 1;
            const size_t w = (size_t)ti * row_words + hrow;
            wk[i] = r.k_new[w];
            wv[i] = r.v_new[w];
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if ((todo >> i) & 1)
                fp8_put_row(r, fp8_readlane64(blk, i), h, __builtin_amdgcn_readlane(off, i), wk[i], wv[i],
                            __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ks_l), i)),
                            __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, vs_l), i)),
                            lane);
        }
    }
}

}  // namespace kvp
