// Paged decode attention for bf16 and FP8 pools with head_dim 128: both
// products on the matrix cores, the online softmax on the vector ALUs.
//
// What is computed is the same as decode.hip (aicassindra.com "GPU paged KV
// cache", "Inside the paged attention kernel"; "PagedAttention, Internals
// First", "02 Block tables"); this file only changes how a gfx950 compute unit
// spends its cycles on it:
//
//   * Scores.  For one (block, KV head) tile the scores of all query heads of
//     the group are S = K Q^T, a 16 x 128 by 128 x G product.  It runs as four
//     v_mfma_f32_16x16x32_bf16: the K tile is the A operand, read straight
//     from HBM (lane l holds token l%16 and eight consecutive dims), the
//     group's queries are the B operand (columns G..15 are zero).  The result
//     leaves lane (r, n) = (l/16, l%16) holding the scores of tokens 4r..4r+3
//     for query head n.
//   * Softmax.  Lane (r, n) keeps the running max and sum of head n over the
//     token positions 4r..4r+3 of every block it walks, so the loop needs no
//     cross-lane reduction.  The max is only moved when a block's scores
//     exceed it by more than 2^kLazy (then the sum and the outputs are
//     rescaled); otherwise exponentials use the old max, which changes no
//     result beyond rounding because output = sum(p v) / sum(p) for any
//     common reference.
//   * Values.  P V runs as eight more MFMAs per tile (see softmax_pv): P is
//     already where the score MFMA left it, and each lane's V operands are
//     repacked from its own V loads (tokens 4r..4r+3, dims 8n..8n+7).
//   * Work.  The tiles of one (sequence, KV head) are walked by one wave at a
//     time.  With partition_size 0 the tiles of the whole batch are cut into
//     equal slices, one per worker wave, and a fix-up merges the (sequence,
//     KV head) pairs that straddle slices (decode_bf16_streamk_kernel); with
//     fixed partitions the partitions go to the same workers whole
//     (decode_partitions_kernel); above 1024 sequences one 4-wave workgroup
//     takes each partition (decode_bf16_mfma_kernel).
//   * Memory.  Block-table entries are fetched with one vector load per 64
//     tiles and read out with readlane; a worker wave holds one tile in
//     registers (fixed partitions: two), and each half of a tile's registers
//     is refilled with the next tile as soon as it has been read, across the
//     end of a walk too: the next piece's table entries are fetched while
//     the current one runs, and its first tiles replace the current walk's
//     last refills.  V tiles of bf16 pools are loaded with the streaming hint
//     (keep_v_cached).
//   * The walk order and all reductions depend only on logical positions, so
//     the output is bitwise independent of where the blocks live.
//   * FP8 pools (E4M3 codes, one fp32 scale per block and KV head for K and
//     one for V): the same kernels with the codes widened to bfloat16 in
//     registers (exact: every E4M3 value is a bfloat16 value).  A block's K
//     scale multiplies its scores; its V scale multiplies the probabilities
//     that enter P V, while the softmax sum takes them unscaled, so
//     out = sum_j p_j sv_j v_j / sum_j p_j is what the dequantized cache gives.
//     Any block size 8..128: with 8-token blocks a tile's two halves are two
//     blocks, and the lanes holding tokens 8..15 (rows r = 2, 3) take the
//     second block's scales.  One tile in registers per worker wave, as for bf16: deeper pipelines
//     (2, 4, 6, 8 FP8 tiles) measured slower on the 8B- and 70B-shaped
//     batches.
#include <math.h>

#include <atomic>

#include "device_common.hpp"
#include "fp8.hpp"
#include "fp8_rows.hpp"
#include "launch.hpp"
#include "split.hpp"
#include "table_index.hpp"

namespace kvp {

namespace {

constexpr int kWaves = 4;
constexpr int kD = 128;            // head_dim this kernel is built for
constexpr int kRC = kD / 8;        // 16-byte chunks per token row (16)
constexpr int kKK = kD / 32;       // MFMA steps over head_dim (4)
constexpr float kLazy = 8.0f;      // log2 headroom before the running max is moved
// Tiles in registers per worker wave.  Balanced split: one (the next tile's
// loads go out as soon as each half of the current one is read).  With two,
// the 8B- and 70B-shaped batches ran 1.5-4% slower for bf16 tiles and 2.5-6%
// slower for FP8 tiles, as a plain gather of the same tiles in the same
// slices does: more requests in flight per wave than the memory system turns
// into bandwidth.  Fixed partitions, whose walks are short: two (one measured
// 2% slower on the long-context batch).
constexpr int kFixupMinWaves = 1024;   // fix-up grids are split over query heads up to this many waves
constexpr int kBalancedDepth = 1;
constexpr int kPartitionDepth = 2;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

template <int CTRL>
__device__ __forceinline__ float bcast(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// lane h of every 16-lane row, to all lanes of that row
template <int H>
__device__ __forceinline__ float row_bcast(float x) {
    return bcast<0x150 + H>(x);
}

__device__ __forceinline__ float safe_ref(float m) { return m == -INFINITY ? 0.0f : m; }

// Value of lane `src` (wave-uniform) in every lane, without going through LDS.
__device__ __forceinline__ float readlane_f(float x, int src) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), src));
}
// Inclusive prefix sum over the wave: within each row of 16 lanes by row
// shifts of 1, 2, 4 and 8 (a lane without a source adds 0), then lane 15's
// sum into rows 1 and 3 and lane 31's into rows 2 and 3 (row broadcasts).
__device__ __forceinline__ int wave_inclusive_sum(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31
    return x;
}
__device__ __forceinline__ int64_t readlane64(int64_t x, int src) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, src);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)x >> 32), src);
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

struct Tile {
    uint4 k[kKK];   // K: token n, dims 32*kk + 8*r .. +8
    uint4 v[4];     // V: token 4*r + i, chunk c
};

// FP8 tile, codes.  K: token n, dims 32r .. 32r+31, so MFMA step kk takes
// dims 32r + 8kk .. +8 (the queries are loaded in the same order).  V: token
// 4r + i, dims 8n .. 8n+7, the dims this lane's outputs stand for.
struct TileF8 {
    uint4 k[2];
    uint2 v[4];
};

template <bool kFp8>
struct TileOf {
    typedef Tile type;
};
template <>
struct TileOf<true> {
    typedef TileF8 type;
};

// Running state of one wave.  The reference max m is the same in all four
// rows (blocks are folded in whole), l is this row's share of the softmax
// sum, and o holds the MFMA accumulators of P V: o[e][j] is the output of
// query head 4r + j, dim 8n + e.
struct State {
    float m, l;            // lane (r, n): head n
    f32x4_t o[8];
};

__device__ __forceinline__ void load_k(Tile& t, const uint4* __restrict__ kt, int k_off) {
#pragma unroll
    for (int kk = 0; kk < kKK; ++kk) t.k[kk] = kt[k_off + kk * 4];
}
// V halves are loaded with the streaming hint unless `keep` (see stream_v in
// WalkCtx); `keep` is wave-uniform, so this is a scalar branch around the loads.
__device__ __forceinline__ void load_v(Tile& t, const uint4* __restrict__ vt, int v_off, bool keep) {
    if (keep) {
#pragma unroll
        for (int i = 0; i < 4; ++i) t.v[i] = vt[v_off + i * kRC];
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) t.v[i] = load_stream(&vt[v_off + i * kRC]);
    }
}
__device__ __forceinline__ void load_k(TileF8& t, const uint4* __restrict__ kt, int k_off) {
    t.k[0] = kt[k_off];
    t.k[1] = kt[k_off + 1];
}
// v_off in 8-byte units; a code row is kD / 8 of them
__device__ __forceinline__ void load_v(TileF8& t, const uint4* __restrict__ vt, int v_off, bool keep) {
    const uint2* p = reinterpret_cast<const uint2*>(vt);
    if (keep) {
#pragma unroll
        for (int i = 0; i < 4; ++i) t.v[i] = p[v_off + i * (kD / 8)];
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) t.v[i] = load_stream(&p[v_off + i * (kD / 8)]);
    }
}

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) {
    bf16x2_t p = {(__bf16)lo, (__bf16)hi};   // round to nearest even
    return __builtin_bit_cast(uint32_t, p);
}

__device__ __forceinline__ bf16x8_t as_operand(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    return __builtin_bit_cast(bf16x8_t, make_uint4(a, b, c, d));
}

// Masking, lazy online softmax with one reference max per head, and P V on
// MFMA for one tile, from its raw scores s (lane (r, n): tokens 4r..4r+3,
// head n) and its V operands: ev[w] / od[w] hold dims 8n + 2w / 8n + 2w + 1 of
// tokens (4r, 4r+1) and (4r+2, 4r+3) as bfloat16 pairs.  vscale multiplies
// the probabilities that enter P V (an FP8 block's V scale, else 1); the
// softmax sum takes them unscaled.
//
// P V is a 16-head x 16-token by 16-token x 128-dim product, split as P =
// P_hi + P_lo (a bfloat16 high part and the bfloat16 of the remainder, so the
// product keeps about 16 bits of P).  It runs as eight
// v_mfma_f32_16x16x32_bf16, one per e = 0..7, whose output column n stands
// for dim 8n + e.  The sum over the 32 positions of the contraction only has
// to pair the same token in A and B, so lane (r, n) puts P_hi and P_lo of
// head n, tokens 4r..4r+3 (already where the score MFMA left them) in its
// eight A positions and dim 8n + e of the same four tokens, twice, in its
// eight B positions.  softmax_pv_core takes the tile once it is masked, with
// vop(e) giving the B operand of the product for dims 8n + e (built from ev /
// od by softmax_pv; built once per tile and shared by several query column
// sets in the prefix walk).
template <int G, class VOp>
__device__ __forceinline__ void softmax_pv_core(State& st, const f32x4_t& s, VOp vop, int r, int n, float sl2,
                                                float vscale) {
    // This row's max of head n.  The reference m is shared by the four rows
    // (their P meet in one MFMA), so it only moves, to the block max over all
    // rows, when some row would exceed it by more than 2^kLazy.
    float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])) * sl2;
    const bool row_need = (n < G) && (mx > st.m + kLazy);
    if (__builtin_amdgcn_ballot_w64(row_need)) {   // rare after the first block
        mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
        mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
        const bool need = (n < G) && (mx > st.m + kLazy);
        const float m_new = need ? mx : st.m;
        const float corr = need ? fast_exp2(st.m - m_new) : 1.0f;   // 0 when nothing was seen yet
        st.l *= corr;
        st.m = m_new;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float cj = __shfl(corr, 4 * r + j, kWave);   // head 4r + j (rows agree)
#pragma unroll
            for (int e = 0; e < 8; ++e) st.o[e][j] *= cj;
        }
    }
    const float neg_ref = -safe_ref(st.m);
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = n < G ? fast_exp2(fmaf(s[i], sl2, neg_ref)) : 0.0f;
    st.l += (p[0] + p[1]) + (p[2] + p[3]);
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] *= vscale;

    const uint32_t h01 = bf16_pair(p[0], p[1]);
    const uint32_t h23 = bf16_pair(p[2], p[3]);
    const uint32_t l01 = bf16_pair(p[0] - bf16_lo(h01), p[1] - bf16_hi(h01));
    const uint32_t l23 = bf16_pair(p[2] - bf16_lo(h23), p[3] - bf16_hi(h23));
    const bf16x8_t pa = as_operand(h01, h23, l01, l23);
#pragma unroll
    for (int e = 0; e < 8; ++e) st.o[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vop(e), st.o[e], 0, 0, 0);
}

template <int G>
__device__ __forceinline__ void softmax_pv(State& st, f32x4_t s, uint32_t (&ev)[4][2], uint32_t (&od)[4][2],
                                           int tok0, int L, int r, int n, float sl2, float vscale) {
    if (tok0 + kTileTokens > L) {   // last, partially filled tile (wave-uniform branch)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (tok0 + 4 * r + i >= L) {
                s[i] = -INFINITY;
                // stale slots may hold NaN; P is 0 there
                const uint32_t keep = (i & 1) ? 0x0000FFFFu : 0xFFFF0000u;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    ev[w][i >> 1] &= keep;
                    od[w][i >> 1] &= keep;
                }
            }
        }
    }

    softmax_pv_core<G>(
        st, s,
        [&](int e) __attribute__((always_inline)) {
            const int w = e >> 1;
            return (e & 1) ? as_operand(od[w][0], od[w][1], od[w][0], od[w][1])
                           : as_operand(ev[w][0], ev[w][1], ev[w][0], ev[w][1]);
        },
        r, n, sl2, vscale);
}

// One bf16 tile: scores on MFMA, then the steps of softmax_pv written out in
// place (with a V scale of 1).  The tile's registers are refilled with the
// next tile as soon as they are consumed: after_k() is called once the K half
// has been read, after_v() once the V half has.  The V operands are already
// in the lane's own V loads and are only repacked.  Kept as one body: with
// softmax_pv called here the bf16 walk took 264 registers instead of 254, so
// a second wave no longer fit on a SIMD beside a worker and the decode-append
// waves of the balanced kernel could not run alongside the workers.
template <int G, class AfterK, class AfterV>
__device__ __forceinline__ void process(State& st, Tile& t, const bf16x8_t (&qb)[kKK], int tok0, int L,
                                        int r, int n, float sl2, AfterK after_k, AfterV after_v) {
    f32x4_t s = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kk = 0; kk < kKK; ++kk)
        s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, t.k[kk]), qb[kk], s, 0, 0, 0);
    // The refills reuse the tile's registers.  An empty asm statement that
    // consumes the results and clobbers memory keeps the reads before it and
    // the refill loads after it.
    asm volatile("" : "+v"(s) : : "memory");
    after_k();

    // dim 8n + 2w (low halves) and 8n + 2w + 1 (high halves) of tokens 4r..4r+3
    uint32_t ev[4][2], od[4][2];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const uint32_t x0 = (&t.v[0].x)[w], x1 = (&t.v[1].x)[w], x2 = (&t.v[2].x)[w], x3 = (&t.v[3].x)[w];
        ev[w][0] = (x0 & 0xFFFFu) | (x1 << 16);
        ev[w][1] = (x2 & 0xFFFFu) | (x3 << 16);
        od[w][0] = (x0 >> 16) | (x1 & 0xFFFF0000u);
        od[w][1] = (x2 >> 16) | (x3 & 0xFFFF0000u);
    }
    asm volatile("" : "+v"(ev[0][0]), "+v"(ev[0][1]), "+v"(ev[1][0]), "+v"(ev[1][1]), "+v"(ev[2][0]), "+v"(ev[2][1]),
                 "+v"(ev[3][0]), "+v"(ev[3][1]), "+v"(od[0][0]), "+v"(od[0][1]), "+v"(od[1][0]), "+v"(od[1][1]),
                 "+v"(od[2][0]), "+v"(od[2][1]), "+v"(od[3][0]), "+v"(od[3][1]) : : "memory");
    after_v();

    if (tok0 + kTileTokens > L) {   // last, partially filled tile (wave-uniform branch)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (tok0 + 4 * r + i >= L) {
                s[i] = -INFINITY;
                // stale slots may hold NaN; P is 0 there
                const uint32_t keep = (i & 1) ? 0x0000FFFFu : 0xFFFF0000u;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    ev[w][i >> 1] &= keep;
                    od[w][i >> 1] &= keep;
                }
            }
        }
    }

    // This row's max of head n.  The reference m is shared by the four rows
    // (their P meet in one MFMA), so it only moves, to the block max over all
    // rows, when some row would exceed it by more than 2^kLazy.
    float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])) * sl2;
    const bool row_need = (n < G) && (mx > st.m + kLazy);
    if (__builtin_amdgcn_ballot_w64(row_need)) {   // rare after the first block
        mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
        mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
        const bool need = (n < G) && (mx > st.m + kLazy);
        const float m_new = need ? mx : st.m;
        const float corr = need ? fast_exp2(st.m - m_new) : 1.0f;   // 0 when nothing was seen yet
        st.l *= corr;
        st.m = m_new;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float cj = __shfl(corr, 4 * r + j, kWave);   // head 4r + j (rows agree)
#pragma unroll
            for (int e = 0; e < 8; ++e) st.o[e][j] *= cj;
        }
    }
    const float neg_ref = -safe_ref(st.m);
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = n < G ? fast_exp2(fmaf(s[i], sl2, neg_ref)) : 0.0f;
    st.l += (p[0] + p[1]) + (p[2] + p[3]);

    const uint32_t h01 = bf16_pair(p[0], p[1]);
    const uint32_t h23 = bf16_pair(p[2], p[3]);
    const uint32_t l01 = bf16_pair(p[0] - bf16_lo(h01), p[1] - bf16_hi(h01));
    const uint32_t l23 = bf16_pair(p[2] - bf16_lo(h23), p[3] - bf16_hi(h23));
    const bf16x8_t pa = as_operand(h01, h23, l01, l23);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        st.o[2 * w] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            pa, as_operand(ev[w][0], ev[w][1], ev[w][0], ev[w][1]), st.o[2 * w], 0, 0, 0);
        st.o[2 * w + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            pa, as_operand(od[w][0], od[w][1], od[w][0], od[w][1]), st.o[2 * w + 1], 0, 0, 0);
    }
}

// One FP8 tile: the codes are widened to bfloat16 operands (two per
// v_cvt_scalef32_pk_bf16_fp8), the K scale multiplies the raw scores and the
// V scale goes to softmax_pv.  For V, v_perm_b32 first gathers byte e of the
// tokens (4r, 4r+1) and of (4r+2, 4r+3) next to each other, so one widening
// yields the bfloat16 pair softmax_pv expects.
template <int G, class AfterK, class AfterV>
__device__ __forceinline__ void process(State& st, TileF8& t, const bf16x8_t (&qb)[kKK], int tok0, int L,
                                        int r, int n, float sl2, float kscale, float vscale, AfterK after_k,
                                        AfterV after_v) {
    f32x4_t s = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kk = 0; kk < kKK; ++kk) {
        const uint32_t d0 = (&t.k[kk >> 1].x)[2 * (kk & 1)];
        const uint32_t d1 = (&t.k[kk >> 1].x)[2 * (kk & 1) + 1];
        const bf16x8_t ka = as_operand(e4m3x2_to_bf16x2<false>(d0), e4m3x2_to_bf16x2<true>(d0),
                                       e4m3x2_to_bf16x2<false>(d1), e4m3x2_to_bf16x2<true>(d1));
        s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qb[kk], s, 0, 0, 0);
    }
    asm volatile("" : "+v"(s) : : "memory");
    after_k();

    uint32_t ev[4][2], od[4][2];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        // bytes 2(w&1), 2(w&1)+1 of word w/2 (dims 8n + 2w, 8n + 2w + 1), interleaved over two tokens
        const uint32_t sel = (w & 1) ? 0x07030602u : 0x05010400u;
        const uint32_t y01 = __builtin_amdgcn_perm((&t.v[1].x)[w >> 1], (&t.v[0].x)[w >> 1], sel);
        const uint32_t y23 = __builtin_amdgcn_perm((&t.v[3].x)[w >> 1], (&t.v[2].x)[w >> 1], sel);
        ev[w][0] = e4m3x2_to_bf16x2<false>(y01);
        od[w][0] = e4m3x2_to_bf16x2<true>(y01);
        ev[w][1] = e4m3x2_to_bf16x2<false>(y23);
        od[w][1] = e4m3x2_to_bf16x2<true>(y23);
    }
    asm volatile("" : "+v"(ev[0][0]), "+v"(ev[0][1]), "+v"(ev[1][0]), "+v"(ev[1][1]), "+v"(ev[2][0]), "+v"(ev[2][1]),
                 "+v"(ev[3][0]), "+v"(ev[3][1]), "+v"(od[0][0]), "+v"(od[0][1]), "+v"(od[1][0]), "+v"(od[1][1]),
                 "+v"(od[2][0]), "+v"(od[2][1]), "+v"(od[3][0]), "+v"(od[3][1]) : : "memory");
    after_v();
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] *= kscale;
    softmax_pv<G>(st, s, ev, od, tok0, L, r, n, sl2, vscale);
}

// End of a walk: lane (r, n) gets the whole softmax sum of head n.
__device__ __forceinline__ float total_l(const State& st) {
    float l = st.l + __shfl_xor(st.l, 16, kWave);
    return l + __shfl_xor(l, 32, kWave);
}

// Everything one wave needs to walk blocks of one (sequence, KV head).
struct WalkCtx {
    const uint4* kpool;
    const uint4* vpool;
    size_t head_off;       // kv * tile chunks
    size_t head_stride;    // chunks between the tiles of consecutive KV heads in a block
    size_t block_stride;   // num_kv_heads * B * 16-byte chunks per row
    uint32_t num_blocks;
    int max_blocks;        // table entries per sequence (the row pitch)
    int row_len;           // entries the walked row pointer can address: max_blocks, or what
                           // follows a shared prefix when the walk starts after it
    bool pair8;            // B = 8: a 16-token tile is two blocks
    int sub_shift;         // B >= 16: log2(B / 16), tiles per block = 1 << sub_shift
    int k_off, v_off;      // this lane's K (16-byte units) / V (16-byte, FP8: 8-byte units) offset in a tile
    int lane, r, n;
    float sl2;
    const float* ksc;      // FP8: scales of KV head kv in block 0; block p's are at p * nkvh
    const float* vsc;
    int nkvh;
    bool keep_v;           // load V with the ordinary (cached) policy, not the streaming hint
};

// Cache policy of a walk's V loads.  K tiles are loaded with the ordinary
// policy and V tiles with the streaming hint: a call reads its K/V once, and
// on MI355X keeping V out of the caches lets the 8B-shaped batch stream at
// 6.05 TB/s instead of 5.1 (the streaming hint on K as well measured slower:
// a K load instruction covers half of each of 16 lines, and a streamed line is
// gone before the instruction for its other half).  The exception is a shared
// prefix, whose blocks every sequence of the group reads in the same call:
// when the block under a walk's first tile sits at the same place in a
// neighbouring sequence's table (the shape of a fork or of a prompt shared
// through a prefix cache), V stays cached.  Only a hint: a neighbour's entry
// past its own length may hold anything and is only compared.
template <bool kFp8>
__device__ __forceinline__ bool keep_v_cached(const DecodeArgs& a, int seq, int tile, const WalkCtx& c) {
    if (kFp8) return true;   // FP8 tiles: the hint measured no different (8B, 70B, long-context batches)
    const int entry = c.pair8 ? 2 * tile : tile >> c.sub_shift;
    const int32_t* t = a.tables + (size_t)seq * a.max_blocks + a.shared_entries + entry;
    const int32_t mine = t[0];
    bool shared = false;
    if (seq > 0) shared = shared || t[-(ptrdiff_t)a.max_blocks] == mine;
    if (seq + 1 < a.num_seqs) shared = shared || t[a.max_blocks] == mine;
    return shared;
}

// The same test for a piece whose first table entries are fetched ahead (lane
// 0 of tv0 holds the entry of its first tile): the neighbours' entries are
// fetched with them, lane 0 the previous sequence's and lane 1 the next one's,
// so the piece starts without a round trip for the test.
template <bool kFp8>
__device__ __forceinline__ int neighbour_entries(const DecodeArgs& a, int seq, int tile, const WalkCtx& c) {
    int x = 0;
    if (!kFp8) {
        const int entry = c.pair8 ? 2 * tile : tile >> c.sub_shift;
        if (c.lane == 0 && seq > 0) x = a.tables[(size_t)(seq - 1) * a.max_blocks + a.shared_entries + entry];
        if (c.lane == 1 && seq + 1 < a.num_seqs) x = a.tables[(size_t)(seq + 1) * a.max_blocks + a.shared_entries + entry];
    }
    return x;
}
template <bool kFp8>
__device__ __forceinline__ bool keep_v_fetched(int tv0, int nb, int seq, int num_seqs) {
    if (kFp8) return true;
    const int mine = __builtin_amdgcn_readlane(tv0, 0);
    return (seq > 0 && __builtin_amdgcn_readlane(nb, 0) == mine) ||
           (seq + 1 < num_seqs && __builtin_amdgcn_readlane(nb, 1) == mine);
}

// kAnyB: the block size comes from the arguments (8..128); otherwise it is 16
// and every block-size field below is a constant the walk folds away.
// kFp8: an FP8 pool.
template <bool kAnyB, bool kFp8 = false>
__device__ __forceinline__ WalkCtx make_ctx(const DecodeArgs& a, int kv) {
    const int B = kAnyB ? a.block_size : kTileTokens;
    constexpr int kRow = kFp8 ? kD / 16 : kRC;   // 16-byte chunks per token row
    WalkCtx c;
    c.lane = threadIdx.x & (kWave - 1);
    c.r = c.lane >> 4;
    c.n = c.lane & 15;
    c.kpool = reinterpret_cast<const uint4*>(a.k_layer);
    c.vpool = reinterpret_cast<const uint4*>(a.v_layer);
    c.head_stride = (size_t)B * kRow;
    c.head_off = (size_t)kv * c.head_stride;
    c.block_stride = (size_t)a.num_kv_heads * ((size_t)B * kRow);
    c.num_blocks = (uint32_t)a.num_blocks;
    c.max_blocks = a.max_blocks;
    c.row_len = a.max_blocks;
    c.pair8 = kAnyB && B == 8;
    c.sub_shift = kAnyB ? 31 - __builtin_clz(B >= kTileTokens ? B / kTileTokens : 1) : 0;
    if constexpr (kFp8) {
        // K: token n, chunks 2r and 2r + 1; V: token 4r + i, 8-byte unit n
        // (rows within the lane's block when B = 8)
        c.k_off = (c.pair8 ? (c.n & 7) : c.n) * kRow + 2 * c.r;
        c.v_off = (c.pair8 ? ((4 * c.r) & 7) : 4 * c.r) * (kD / 8) + c.n;
        c.ksc = a.k_scale + kv;
        c.vsc = a.v_scale + kv;
        c.nkvh = a.num_kv_heads;
    } else {
        // K: token n, chunk 4*kk + r; V: token 4r + i, chunk n (rows within the lane's block when B = 8)
        c.k_off = (c.pair8 ? (c.n & 7) : c.n) * kRC + c.r;
        c.v_off = (c.pair8 ? ((4 * c.r) & 7) : 4 * c.r) * kRC + c.n;
        c.ksc = c.vsc = nullptr;
        c.nkvh = 0;
    }
    c.sl2 = a.scale_log2;
    c.keep_v = false;
    return c;
}

// B operand: the group's query heads as columns, zero beyond G.  Step kk
// takes dims 32kk + 8r .. +8 (bf16 tiles) or 32r + 8kk .. +8 (FP8 tiles), as
// the K operand does.
template <int G, bool kFp8 = false>
__device__ __forceinline__ void load_q(bf16x8_t (&qb)[kKK], const DecodeArgs& a, int seq, int kv, const WalkCtx& c) {
    const uint4* qrow = reinterpret_cast<const uint4*>(a.q) + ((size_t)seq * a.num_q_heads + (size_t)kv * G) * kRC;
#pragma unroll
    for (int kk = 0; kk < kKK; ++kk) {
        uint4 x = make_uint4(0u, 0u, 0u, 0u);
        if (c.n < G) x = qrow[c.n * kRC + (kFp8 ? 4 * c.r + kk : kk * 4 + c.r)];
        qb[kk] = __builtin_bit_cast(bf16x8_t, x);
    }
}

__device__ __forceinline__ void init_state(State& st) {
    st.m = -INFINITY;
    st.l = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) st.o[e] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
}

// Decode append inside the walk: the block holding position L - 1 (the token
// written this step) takes row j = (L - 1) % B from the new K/V row instead of
// the pool.  The row is stored into the pool by separate waves of the same
// launch (append_scatter_waves): stores share the in-order memory counter with
// loads, so a store from this wave would make its next waits cover it too.
// Whatever this wave reads for row j is replaced, so it does not matter
// whether it sees the old or the new row.
struct AppendRow {
    bool active;
    bool store;           // FP8 pools: the walk also stores the row (codes and, opening a block, its scales)
    int tok0;             // first token of the block holding position L - 1
    int j;                // (L - 1) % 16: the row within its 16-token tile
    int brow;             // (L - 1) % B: the row within its block
    bool opens;           // (L - 1) % B == 0: the row is row 0 of its block
    const uint4* krow;    // the new K row (16 chunks)
    const uint4* vrow;
};

// Lane (r, n) holds K token n, chunks 4kk + r, and V tokens 4r + i, chunk n.
__device__ __forceinline__ void append_into(Tile& t, const AppendRow& app, const uint4 (&nk)[kKK], uint4 nv,
                                            const WalkCtx& c) {
    if (c.n == app.j) {
#pragma unroll
        for (int kk = 0; kk < kKK; ++kk) t.k[kk] = nk[kk];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (4 * c.r + i == app.j) t.v[i] = nv;
}

// FP8 tiles: the new row is quantized here exactly as the pool-side waves
// quantize it (fp8_store_row: lane l takes dims 2l and 2l + 1 of the bf16 row,
// kw for K and vw for V, so both sides compute the same codes and scales),
// then the codes move to the lanes that hold the row in the tile layout: K
// dims 32r + 4m .. +3 (m = 0..7) from lane 16r + 2m, V dims 8n .. 8n+7 from
// lanes 4n and 4n + 2.  When the row is row 0 of its block (app.opens) it
// alone sets the block's scales, which then replace the scales read for the
// block.  kscale / vscale are the scales of the block holding the row (with
// 8-token blocks, the tile's half).  With app.store the wave also stores the
// row's codes at kdst / vdst (lane l: dims 2l, 2l + 1, as fp8_store_row) and,
// opening the block, its scales at ksd / vsd: the one wave that walks a (sequence,
// KV head)'s last tile is the pool side of its append.
__device__ __forceinline__ void append_into_fp8(TileF8& t, const AppendRow& app, uint32_t kw, uint32_t vw,
                                                const WalkCtx& c, float& kscale, float& vscale, uint16_t* kdst,
                                                uint16_t* vdst, float* ksd, float* vsd) {
    if (app.opens) {   // wave-uniform
        kscale = e4m3_block_scale(wave_max(abs_max2(kw, 0.0f)));
        vscale = e4m3_block_scale(wave_max(abs_max2(vw, 0.0f)));
    }
    const uint32_t k2 = bf16x2_to_e4m3x2(kw, kscale);   // codes of dims 2l, 2l + 1
    const uint32_t v2 = bf16x2_to_e4m3x2(vw, vscale);
    if (app.store) {   // wave-uniform
        kdst[c.lane] = (uint16_t)k2;
        vdst[c.lane] = (uint16_t)v2;
        if (app.opens && c.lane == 0) {
            *ksd = kscale;
            *vsd = vscale;
        }
    }
    const uint32_t k4 = k2 | ((uint32_t)__shfl_down((int)k2, 1, kWave) << 16);   // even lanes: dims 2l .. 2l+3
    const uint32_t v4 = v2 | ((uint32_t)__shfl_down((int)v2, 1, kWave) << 16);
    uint32_t kd[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) kd[m] = (uint32_t)__shfl((int)k4, 16 * c.r + 2 * m, kWave);
    const uint2 vd = make_uint2((uint32_t)__shfl((int)v4, 4 * c.n, kWave), (uint32_t)__shfl((int)v4, 4 * c.n + 2, kWave));
    if (c.n == app.j) {
        t.k[0] = make_uint4(kd[0], kd[1], kd[2], kd[3]);
        t.k[1] = make_uint4(kd[4], kd[5], kd[6], kd[7]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (4 * c.r + i == app.j) t.v[i] = vd;
}

// Table entries of tile e (16 tokens) of a sequence whose table row is `row`
// (c.row_len entries from there): for B >= 16 the block holding it (entry
// e / (B/16)); for B = 8 the two blocks holding its halves (entries 2e and
// 2e + 1; the second is not read when it lies past the row: the tile is then
// the row's last one and its second half is never used).
__device__ __forceinline__ int2 tile_entries(const int32_t* row, int e, bool valid, const WalkCtx& c) {
    int2 tv = make_int2(0, 0);
    if (valid) {
        tv.x = row[tile_first_entry(e, c.pair8, c.sub_shift)];
        if (tile_has_second_entry(e, c.row_len, c.pair8)) tv.y = row[2 * e + 1];
    }
    return tv;
}

// The walk that follows on the same wave, when its first table entries are
// already in registers: the last refills of a walk then fetch its first tiles
// instead of repeating a tile, so that it starts with them in flight.
struct NextWalk {
    bool valid;
    int tv0, tv1;          // lane j: table entries of its tile j (tv1: B = 8's second block)
    int e0;                // its first 16-token tile in its sequence
    size_t head_off;       // its KV head's offset in a block (16-byte units)
    int count;             // its tiles (at least 1)
};

__device__ __forceinline__ NextWalk no_next_walk() {
    NextWalk n;
    n.valid = false;
    n.tv0 = n.tv1 = n.e0 = 0;
    n.head_off = 0;
    n.count = 1;
    return n;
}

// Walk nk blocks of one (sequence, KV head): logical blocks b0 + stride*k,
// k = 0..nk-1, whose table entries start at trow (= row + b0).
//
// Table entries come 64 at a time from one vector load.  Within such a chunk
// D tiles are held in registers (tt, owned by the caller): while block k is
// computed, blocks k+1 .. k+D-1 are in flight, and block k's registers are
// refilled with block k+D as soon as each half has been read.  Every tile
// load is issued unconditionally and in the order the tiles are consumed, so
// the hardware's in-order load counter lets each block wait for its own tile
// only.  Past the end of a chunk a refill fetches the chunk's last tile again
// (an L2 hit), except past the end of the walk when the next walk of this
// wave is known (nxt): then the refills fetch that walk's first D tiles, and
// the caller starts it with primed = true (its tiles already requested).
//
// FP8 tiles also need their block scales: lane k of the chunk loads those of
// tile k before the first tiles are requested, and tile k reads them from
// lane k.
template <int G, int D, bool kFp8, bool kKeepV>
__device__ __forceinline__ void walk_policy(State& st, typename TileOf<kFp8>::type (&tt)[D], bool primed,
                                            const bf16x8_t (&qb)[kKK], const int32_t* row, int stride, int nk,
                                            int b0, int L, const WalkCtx& c, const AppendRow& app, bool have_first,
                                            int tv0_first, int tv1_first, const NextWalk& nxt) {
    // Tile k of the current chunk (tile b0 + (k0 + k) * stride of the sequence).
    // Each lane addresses its own rows: for B = 8 the K rows of tokens 8..15 and
    // the V rows of lanes r >= 2 come from the second block.
    int k0 = 0;
    constexpr int kRowChunks = kFp8 ? kD / 16 : kRC;   // 16-byte chunks per token row
    auto ptrs_of = [&](uint32_t p0, uint32_t p1, int e, size_t head_off, const uint4*& kt, const uint4*& vt) {
        p0 = p0 < c.num_blocks ? p0 : c.num_blocks - 1;   // stay inside the pool whatever the table says
        if (c.pair8) {
            p1 = p1 < c.num_blocks ? p1 : c.num_blocks - 1;
            kt = c.kpool + (size_t)(c.n < 8 ? p0 : p1) * c.block_stride + head_off;
            vt = c.vpool + (size_t)(c.r < 2 ? p0 : p1) * c.block_stride + head_off;
        } else {
            const size_t base = (size_t)p0 * c.block_stride + head_off +
                                (size_t)(e & ((1 << c.sub_shift) - 1)) * (kTileTokens * kRowChunks);
            kt = c.kpool + base;
            vt = c.vpool + base;
        }
    };
    auto tile_ptrs = [&](int tv0, int tv1, int k, const uint4*& kt, const uint4*& vt) {
        ptrs_of((uint32_t)__builtin_amdgcn_readlane(tv0, k), c.pair8 ? (uint32_t)__builtin_amdgcn_readlane(tv1, k) : 0u,
                b0 + (k0 + k) * stride, c.head_off, kt, vt);
    };
    // tile j of the next walk
    auto next_ptrs = [&](int j, const uint4*& kt, const uint4*& vt) {
        ptrs_of((uint32_t)__builtin_amdgcn_readlane(nxt.tv0, j),
                c.pair8 ? (uint32_t)__builtin_amdgcn_readlane(nxt.tv1, j) : 0u, nxt.e0 + j, nxt.head_off, kt, vt);
    };
    // the block holding row j of tile k names a block of the pool
    auto row_in_pool = [&](int tv0, int tv1, int k, int j) -> bool {
        const int tv = (c.pair8 && j >= 8) ? tv1 : tv0;
        return (uint32_t)__builtin_amdgcn_readlane(tv, k) < c.num_blocks;
    };
    uint4 new_k[kKK], new_v;   // the appended row, loaded once the last chunk's first tiles are in flight
    uint32_t new_kw = 0, new_vw = 0;   // FP8: dims 2l, 2l + 1 of the appended row
    for (k0 = 0; k0 < nk; k0 += 64) {
        const int nc = min(64, nk - k0);
        const bool last_chunk = k0 + 64 >= nk;
        const int nc_pad = (nc + D - 1) / D * D;   // tiles the loop below runs, masked ones included
        // the first chunk's entries may have been fetched ahead (entries past nc are never read)
        const int2 tvp = (k0 == 0 && have_first) ? make_int2(tv0_first, tv1_first)
                                                 : tile_entries(row, b0 + (k0 + c.lane) * stride, c.lane < nc, c);
        const int tv0 = tvp.x, tv1 = tvp.y;
        float ks_l = 1.0f, vs_l = 1.0f, ks_l1 = 1.0f, vs_l1 = 1.0f;
        if constexpr (kFp8) {
            if (c.lane < nc) {
                uint32_t p = (uint32_t)tv0;
                p = p < c.num_blocks ? p : c.num_blocks - 1;
                ks_l = c.ksc[(size_t)p * c.nkvh];
                vs_l = c.vsc[(size_t)p * c.nkvh];
                if (c.pair8) {   // tokens 8..15 of the tile
                    uint32_t p1 = (uint32_t)tv1;
                    p1 = p1 < c.num_blocks ? p1 : c.num_blocks - 1;
                    ks_l1 = c.ksc[(size_t)p1 * c.nkvh];
                    vs_l1 = c.vsc[(size_t)p1 * c.nkvh];
                }
            }
            asm volatile("" : : : "memory");
        }
        const uint4 *kt, *vt;
        if (!(k0 == 0 && primed)) {
#pragma unroll
            for (int s = 0; s < D; ++s) {
                tile_ptrs(tv0, tv1, min(s, nc - 1), kt, vt);
                load_k(tt[s], kt, c.k_off);
                asm volatile("" : : : "memory");
                load_v(tt[s], vt, c.v_off, kKeepV);
                asm volatile("" : : : "memory");
            }
        }
        if (app.active && last_chunk) {
            if constexpr (kFp8) {
                new_kw = reinterpret_cast<const uint32_t*>(app.krow)[c.lane];
                new_vw = reinterpret_cast<const uint32_t*>(app.vrow)[c.lane];
            } else {
#pragma unroll
                for (int kk = 0; kk < kKK; ++kk) new_k[kk] = app.krow[4 * kk + c.r];
                new_v = app.vrow[c.n];
            }
        }
        const bool to_next = last_chunk && nxt.valid;
        for (int k = 0; k < nc; k += D) {
#pragma unroll
            for (int s = 0; s < D; ++s) {
                // tt[s] holds block k + s; it is refilled with block k + s + D.
                // Past the end a block is a repeat, given a first token of L
                // so that every position is masked and it adds exact zeros;
                // running it anyway keeps the loads of every path equal.  The
                // refills of the last D slots fetch the next walk's tiles 0..D-1.
                const int idx = k + s + D;
                if (to_next && idx >= nc_pad)
                    next_ptrs(min(idx - nc_pad, nxt.count - 1), kt, vt);
                else
                    tile_ptrs(tv0, tv1, min(idx, nc - 1), kt, vt);
                __builtin_amdgcn_sched_barrier(0);
                const int tok = k + s < nc ? (b0 + (k0 + k + s) * stride) * kTileTokens : L;
                if constexpr (kFp8) {
                    const int ks = min(k + s, nc - 1);
                    float ksc = readlane_f(ks_l, ks), vsc = readlane_f(vs_l, ks);
                    float ksc1 = ksc, vsc1 = vsc;   // B = 8: the scales of tokens 8..15
                    if (c.pair8) {
                        ksc1 = readlane_f(ks_l1, ks);
                        vsc1 = readlane_f(vs_l1, ks);
                    }
                    if (app.active && tok == app.tok0 && row_in_pool(tv0, tv1, k + s, app.j)) {
                        const bool hi = c.pair8 && app.j >= 8;   // B = 8: the tile's second block
                        uint16_t *kd = nullptr, *vd = nullptr;
                        float *ksd = nullptr, *vsd = nullptr;
                        if (app.store) {
                            const size_t blk = (uint32_t)__builtin_amdgcn_readlane(hi ? tv1 : tv0, k + s);
                            // 16-byte chunks to the block's rows of this head, then 64 code pairs a row
                            const size_t at = (blk * c.block_stride + c.head_off) * 8 + (size_t)app.brow * (kD / 2);
                            kd = reinterpret_cast<uint16_t*>(const_cast<uint4*>(c.kpool)) + at;
                            vd = reinterpret_cast<uint16_t*>(const_cast<uint4*>(c.vpool)) + at;
                            ksd = const_cast<float*>(c.ksc) + blk * c.nkvh;
                            vsd = const_cast<float*>(c.vsc) + blk * c.nkvh;
                        }
                        if (hi)
                            append_into_fp8(tt[s], app, new_kw, new_vw, c, ksc1, vsc1, kd, vd, ksd, vsd);
                        else
                            append_into_fp8(tt[s], app, new_kw, new_vw, c, ksc, vsc, kd, vd, ksd, vsd);
                    }
                    // lane (r, n) holds the scores and probabilities of tokens 4r .. 4r+3
                    const bool second = c.pair8 && c.r >= 2;
                    process<G>(st, tt[s], qb, tok, L, c.r, c.n, c.sl2, second ? ksc1 : ksc, second ? vsc1 : vsc,
                               [&] { load_k(tt[s], kt, c.k_off); }, [&] { load_v(tt[s], vt, c.v_off, kKeepV); });
                } else {
                    // wave-uniform: the tile holding the new token; a table entry outside
                    // the pool gets no write (as the scatter skips such a slot)
                    if (app.active && tok == app.tok0 && row_in_pool(tv0, tv1, k + s, app.j)) {
                        append_into(tt[s], app, new_k, new_v, c);
                    }
                    process<G>(st, tt[s], qb, tok, L, c.r, c.n, c.sl2,
                               [&] { load_k(tt[s], kt, c.k_off); }, [&] { load_v(tt[s], vt, c.v_off, kKeepV); });
                }
            }
        }
    }
}

// The walk with the cache policy of its V loads fixed at compile time: a
// runtime choice inside the loop put a branch around every V refill, and that
// cost 1.3 us per call on the 8B-shaped batch and 10 us on the 70B-shaped one.
// Returns whether tt now holds the first tiles of nxt.
template <int G, int D, bool kFp8>
__device__ __forceinline__ bool walk(State& st, typename TileOf<kFp8>::type (&tt)[D], bool primed,
                                     const bf16x8_t (&qb)[kKK], const int32_t* row, int stride, int nk, int b0,
                                     int L, const WalkCtx& c, const AppendRow& app, bool have_first = false,
                                     int tv0_first = 0, int tv1_first = 0, const NextWalk& nxt = no_next_walk()) {
    if (kFp8 || c.keep_v)
        walk_policy<G, D, kFp8, true>(st, tt, primed, qb, row, stride, nk, b0, L, c, app, have_first, tv0_first,
                                      tv1_first, nxt);
    else
        walk_policy<G, D, kFp8, false>(st, tt, primed, qb, row, stride, nk, b0, L, c, app, have_first, tv0_first,
                                       tv1_first, nxt);
    return nk > 0 && nxt.valid;
}


template <int G, bool kAnyB, bool kFp8>
__global__ __launch_bounds__(kWaves * kWave) void decode_bf16_mfma_kernel(DecodeArgs a) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int part = blockIdx.x;
    const int kv = blockIdx.y;
    const int seq = blockIdx.z;

    int L = a.lens[seq];
    L = L < 0 ? 0 : (L > a.max_context ? a.max_context : L);
    L = __builtin_amdgcn_readfirstlane(L);
    const int nparts = L == 0 ? 1 : (L + a.part_tokens - 1) / a.part_tokens;
    if (part >= nparts) return;
    const int nblk = (L + kTileTokens - 1) / kTileTokens;   // 16-token tiles
    const int bpp = a.part_tokens / kTileTokens;
    const int b_begin = part * bpp;
    const int b_end = min(nblk, b_begin + bpp);

    WalkCtx c = make_ctx<kAnyB, kFp8>(a, kv);
    c.keep_v = keep_v_cached<kFp8>(a, seq, b_begin, c);
    const int r = c.r, n = c.n;
    bf16x8_t qb[kKK];
    load_q<G, kFp8>(qb, a, seq, kv, c);
    State st;
    init_state(st);

    const int first = b_begin + wave;
    const int nk = first < b_end ? (b_end - first + kWaves - 1) / kWaves : 0;
    AppendRow none;
    none.active = false;
    none.store = false;
    none.opens = false;
    none.brow = 0;
    none.krow = none.vrow = nullptr;
    typename TileOf<kFp8>::type tt[2];
    walk<G, 2, kFp8>(st, tt, false, qb, a.tables + (size_t)seq * a.max_blocks, kWaves, nk, first, L, c, none);
    const float l_tot = total_l(st);

    // waves of the workgroup merge through LDS
    __shared__ float sm_m[kWaves][G];
    __shared__ float sm_l[kWaves][G];
    __shared__ float sm_acc[kWaves][G][kD];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int h = 4 * r + j;
        if (h < G) {
#pragma unroll
            for (int e = 0; e < 8; ++e) sm_acc[wave][h][n * 8 + e] = st.o[e][j];
        }
    }
    if (r == 0 && n < G) {
        sm_m[wave][n] = st.m;
        sm_l[wave][n] = l_tot;
    }
    __syncthreads();

    const int hq0 = kv * G;
    for (int it = threadIdx.x; it < G * (kD / 2); it += kWaves * kWave) {
        const int h = it / (kD / 2);
        const int d = (it - h * (kD / 2)) * 2;
        float M = sm_m[0][h];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sm_m[w][h]);
        const float Ms = safe_ref(M);
        float den = 0.0f, n0 = 0.0f, n1 = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float f = fast_exp2(sm_m[w][h] - Ms);
            den = fmaf(sm_l[w][h], f, den);
            n0 = fmaf(sm_acc[w][h][d], f, n0);
            n1 = fmaf(sm_acc[w][h][d + 1], f, n1);
        }
        const size_t row = (size_t)seq * a.num_q_heads + hq0 + h;
        if (nparts == 1) {
            const float o0 = den > 0.0f ? n0 / den : 0.0f;
            const float o1 = den > 0.0f ? n1 / den : 0.0f;
            reinterpret_cast<uint32_t*>(a.out)[(row * kD + d) / 2] = pack_bf16x2(o0, o1);
        } else {
            const size_t slot = row * a.max_parts + part;
            reinterpret_cast<float2*>(a.ws_acc)[(slot * kD + d) / 2] = make_float2(n0, n1);
            if (d == 0) reinterpret_cast<float2*>(a.ws_ml)[slot] = make_float2(M, den);
        }
    }
}

// ---------------------------------------------------------------------------
// Balanced split ("stream-K"): the tiles of all (sequence, KV head) pairs are
// numbered t = 0..T-1 in (sequence, KV head, block) order and worker w (one
// wave) takes the contiguous slice [w*T/W, (w+1)*T/W).  Every worker moves
// the same number of bytes, so none waits for a long sequence at the end.
// A (sequence, KV head) whose tiles all fall in one slice is written straight
// to the output; one split over several slices leaves one fp32 partial state
// per slice (at most two per worker: its first and its last piece) that the
// fix-up kernel merges.
// ---------------------------------------------------------------------------

__device__ __forceinline__ int clamp_len(int L, int max_context) {
    return L < 0 ? 0 : (L > max_context ? max_context : L);
}

// floor(num / den) for 0 <= num < 2^31, 0 < den < 2^31 and a quotient below
// 2^20: the float product with v_rcp_f32's reciprocal (within one ulp) is
// within 2^-21.4 relative, so less than one, of the quotient, and one step
// corrects its truncation.  A float multiply and a check where a double
// division is a dozen dependent instructions, on every worker's start.
__device__ __forceinline__ int div_small(int64_t num, int64_t den) {
    int q = (int)((float)num * __builtin_amdgcn_rcpf((float)den));
    if ((int64_t)q * den > num) {
        --q;
    } else if ((int64_t)(q + 1) * den <= num) {
        ++q;
    }
    return q;
}

// Tokens of sequence i that the balanced walk covers: its context past a
// shared prefix (all of it when there is none).
__device__ __forceinline__ int walk_len(const DecodeArgs& a, int i) {
    const int L = clamp_len(a.lens[i], a.max_context) - a.shared_tiles * kTileTokens;
    return L > 0 ? L : 0;
}

// The raw lengths of every chunk of 64 sequences (lane l of chunk c holds
// sequence 64 c + l; lanes past the batch read its last sequence), all loaded
// before any is used, so that the chunks share one memory round trip: a
// guarded load whose value is used at once is waited for chunk by chunk.
template <int N>
__device__ __forceinline__ void load_chunk_lens(const DecodeArgs& a, int S, int nchunks, int lane, int (&raw)[N]) {
#pragma unroll
    for (int ch = 0; ch < N; ++ch) raw[ch] = ch < nchunks ? a.lens[min(ch * kWave + lane, S - 1)] : 0;
}

// Table row of sequence i from the first tile the balanced walk covers.
__device__ __forceinline__ const int32_t* walk_row(const DecodeArgs& a, int i) {
    return a.tables + (size_t)i * a.max_blocks + a.shared_entries;
}

// Partial state of one (sequence, KV head) piece: the unnormalised output of
// each head, then m and l of each head, padded so every record starts on a
// 16-byte boundary.
template <int G>
__host__ __device__ constexpr int record_floats() {
    return G * kD + ((2 * G + 3) / 4) * 4;
}

template <int G>
__device__ __forceinline__ float* record_ptr(const DecodeArgs& a, int64_t slot) {
    return a.ws_acc + slot * (int64_t)record_floats<G>();
}

// Decode append, the pool side: workgroups past the workers copy each
// sequence's new K/V row to position L - 1 of its table (the slot of "The
// write path", computed here from the table and the length).  A block index
// outside the pool is skipped, as by the scatter.  Items are numbered
// ((seq * 2 + {K,V}) * Hkv + head) * kRC + chunk, one 16-byte chunk each.
__device__ __forceinline__ void append_scatter_waves(const DecodeArgs& a, int64_t x, int64_t nx) {
    // item ((seq * 2 + which) * Hkv + h) * kRC + chunk, in 32 bits (at most 1024 sequences);
    // block sizes are powers of two
    static_assert(kRC == 16, "a row is 16 chunks of 16 bytes");
    const int H = a.num_kv_heads;
    const int bshift = __builtin_ctz((unsigned)a.block_size);
    const int items = a.num_seqs * 2 * H * kRC;
    for (int item = (int)x * kWave + (int)threadIdx.x; item < items; item += (int)nx * kWave) {
        const int ch = item & (kRC - 1);
        const int q = (item >> 4) / H;   // seq * 2 + which (kRC = 16 chunks a row)
        const int h = (item >> 4) - q * H;
        const int which = q & 1;
        const int64_t i = q >> 1;
        const int L = clamp_len(a.lens[i], a.max_context);
        if (L == 0) continue;
        const int pos = L - 1;
        const int64_t block = a.tables[i * (int64_t)a.max_blocks + (pos >> bshift)];
        if (block < 0 || block >= a.num_blocks) continue;
        const int64_t dst = ((block * H + h) * a.block_size + (pos & (a.block_size - 1))) * kRC + ch;
        const int64_t src = (i * a.num_kv_heads + h) * kRC + ch;
        const uint4* from = reinterpret_cast<const uint4*>(which == 0 ? a.k_append : a.v_append);
        uint4* to = const_cast<uint4*>(reinterpret_cast<const uint4*>(which == 0 ? a.k_layer : a.v_layer));
        to[dst] = from[src];
    }
}

// Other rows of the step (reshape_and_cache of rows_k / rows_v to
// rows_slots, e.g. a prefill chunk of a sequence outside the batch), stored by
// nx more waves of the balanced launch: wave x takes rows x, x + nx, ...; a
// row's K and V chunks, numbered ({K,V} * Hkv + head) * 16 + chunk, go out
// kRowChunks per lane per round, the round's loads all in flight before its
// stores, and the next row's slot is read while this one moves.  Block sizes
// are powers of two, so the slot splits with shifts (a 64-bit division per
// chunk on these waves slowed the walk beside them by 8 %).  A slot outside
// the pool is skipped.  The caller guarantees that no slot lies in a block
// this launch's attention reads.
constexpr int kRowChunks = 4;

__device__ __forceinline__ void rows_scatter_waves(const DecodeArgs& a, int64_t x, int64_t nx) {
    const int lane = threadIdx.x;
    const int per_head = a.num_kv_heads * kRC;
    const int per_token = 2 * per_head;
    const int bshift = __builtin_ctz((unsigned)a.block_size);
    const int64_t num_slots = (int64_t)a.num_blocks << bshift;
    const uint4* ksrc = reinterpret_cast<const uint4*>(a.rows_k);
    const uint4* vsrc = reinterpret_cast<const uint4*>(a.rows_v);
    uint4* kdst = const_cast<uint4*>(reinterpret_cast<const uint4*>(a.k_layer));
    uint4* vdst = const_cast<uint4*>(reinterpret_cast<const uint4*>(a.v_layer));
    int64_t next = x < a.num_rows ? a.rows_slots[x] : -1;
    for (int64_t t = x; t < a.num_rows; t += nx) {
        const int64_t slot = next;   // wave-uniform
        next = t + nx < a.num_rows ? a.rows_slots[t + nx] : -1;
        if (slot < 0 || slot >= num_slots) continue;
        const int64_t block = slot >> bshift;
        // chunk (h, c) of the row goes to ((block * Hkv + h) * B + offset) * 16 + c
        const int64_t row0 = (((block * a.num_kv_heads) << bshift) + (slot - (block << bshift))) * kRC;
        const int64_t src0 = t * per_head;
        for (int i0 = 0; i0 < per_token; i0 += kWave * kRowChunks) {
            // loads unconditional (a lane past the row reads its last chunk
            // again and stores nothing), so a round's loads are all in flight;
            // four named chunks, not an array: an array here was placed in LDS
            // by the compiler, each load waited for and copied there
            struct Chunk {
                uint4 v;
                int64_t dst;   // -1: nothing to store
                bool is_v;
            };
            auto load = [&](int u) __attribute__((always_inline)) {
                const int item = i0 + u * kWave + lane;
                const int it = item < per_token ? item : per_token - 1;
                Chunk ch;
                ch.is_v = it >= per_head;
                const int rem = it - (ch.is_v ? per_head : 0);
                ch.dst = item < per_token ? row0 + ((int64_t)(rem >> 4) << (bshift + 4)) + (rem & (kRC - 1)) : -1;
                ch.v = (ch.is_v ? vsrc : ksrc)[src0 + rem];
                return ch;
            };
            auto store = [&](const Chunk& ch) __attribute__((always_inline)) {
                if (ch.dst >= 0) (ch.is_v ? vdst : kdst)[ch.dst] = ch.v;
            };
            static_assert(kRowChunks == 4, "four named chunks");
            const Chunk c0 = load(0), c1 = load(1), c2 = load(2), c3 = load(3);
            asm volatile("" ::: "memory");   // the round's loads all issued before its first store
            store(c0);
            store(c1);
            store(c2);
            store(c3);
        }
    }
}

// Other rows of the step on an FP8 pool (reshape_and_cache of rows_k /
// rows_v to rows_slots with the block scale rule), stored by nx more waves of
// the balanced launch: wave x takes the (16-token chunk, KV head) items x,
// x + nx, ... of the rows (fp8_store_chunk: a block opened by these rows gets
// its scales and all its rows' codes from the wave holding its row 0, any
// other row is quantized with the stored scale).  Bitwise the scatter
// kernels' result; the caller guarantees that no slot lies in a block this
// launch's attention reads or appends to.
__device__ __forceinline__ void fp8_rows_waves(const DecodeArgs& a, int64_t x, int64_t nx) {
    Fp8Rows r;
    r.slots = a.rows_slots;
    r.T = a.num_rows;
    r.k_new = reinterpret_cast<const uint32_t*>(a.rows_k);
    r.v_new = reinterpret_cast<const uint32_t*>(a.rows_v);
    r.k_codes = const_cast<uint16_t*>(reinterpret_cast<const uint16_t*>(a.k_layer));
    r.v_codes = const_cast<uint16_t*>(reinterpret_cast<const uint16_t*>(a.v_layer));
    r.k_scale = const_cast<float*>(a.k_scale);
    r.v_scale = const_cast<float*>(a.v_scale);
    r.B = a.block_size;
    r.H = a.num_kv_heads;
    r.num_slots = (int64_t)a.num_blocks * a.block_size;
    const int64_t items = (a.num_rows + 15) / 16 * a.num_kv_heads;
    const bool narrow = items < ((int64_t)1 << 31);   // the usual case: a 32-bit division
    for (int64_t item = x; item < items; item += nx) {
        const int64_t c = narrow ? (int64_t)((uint32_t)item / (uint32_t)r.H) : item / r.H;   // 16-token chunk
        fp8_store_chunk(r, c * 16, (int)(item - c * r.H), threadIdx.x);
    }
}

// ---------------------------------------------------------------------------
// Shared prefix (paged_attention_decode_shared).  The caller's block manager
// knows that the first shared_tiles table entries of every sequence name the
// same blocks (a common prompt: [KVC] "Prefix sharing, reference counts, and
// copy-on-write", [PIF] "03 Sharing via copy-on-write"), so each (block, KV
// head) tile of the prefix is read once for sixteen query columns instead of
// once per sequence: the G query heads of 16 / G consecutive sequences fill
// the score MFMA's sixteen columns and the P V MFMA's sixteen rows, which one
// sequence's G heads leave mostly zero.  Wave (column block qb, KV head kv,
// part p) walks prefix tiles [p PT, (p + 1) PT) of sequence 0's table row and
// leaves each column's (m, l, unnormalised output) in slot p of the prefix
// states; the fix-up merges them with the balanced walk of what follows the
// prefix.  The prefix waves are workgroups of the balanced kernel's own
// launch, past its workers, so the prefix walk, served mostly from L2, runs
// beside the walk of the private tiles, served from HBM; prefix wave idx
// takes KV head idx mod H_kv, so with eight KV heads the waves of one XCD
// share one head's prefix tiles in its L2.
// ---------------------------------------------------------------------------

// Finished states a worker keeps in LDS instead of storing them at once.  A
// worker's stores and its loads share one in-order counter, so a store issued
// between two walks holds up the next walk's tile waits until it has
// completed; states of walks that another walk of the same worker follows
// are therefore parked here and stored when the worker's work is done.  Only
// lanes 16 * ceil(G / 4) and up hold no head's accumulators; (m, l) of head n
// sit in lane n.  `tag` says where the state goes (kernel-specific).
template <int G, int kSlots>
struct Parked {
    static constexpr int kLanes = 16 * ((G + 3) / 4);
    f32x4_t o[kSlots][8][kLanes];
    float2 ml[kSlots][16];
    int4 tag[kSlots];

    __device__ __forceinline__ void put(int i, const State& st, float l_tot, int4 t, int lane) {
        if (lane < kLanes) {
#pragma unroll
            for (int e = 0; e < 8; ++e) o[i][e][lane] = st.o[e];
        }
        if (lane < 16) ml[i][lane] = make_float2(st.m, l_tot);
        if (lane == 0) tag[i] = t;
    }
    // the state (with its whole softmax sum in l) and the tag, wave-uniform
    __device__ __forceinline__ int4 get(int i, State& st, int lane) const {
#pragma unroll
        for (int e = 0; e < 8; ++e) st.o[e] = lane < kLanes ? o[i][e][lane] : f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        const float2 v = lane < 16 ? ml[i][lane] : make_float2(0.0f, 0.0f);
        st.m = v.x;
        st.l = v.y;
        const int4 t = tag[i];
        return make_int4(__builtin_amdgcn_readfirstlane(t.x), __builtin_amdgcn_readfirstlane(t.y),
                         __builtin_amdgcn_readfirstlane(t.z), __builtin_amdgcn_readfirstlane(t.w));
    }
};
// parked states per worker: the balanced split (a few walks per worker), and
// the fixed partitions (a few more, 16 KiB of LDS per worker)
constexpr int kParkedPieces = 3;
template <int G>
constexpr int parked_partitions() { return 16384 / (16 * ((G + 3) / 4) * 128); }

// The walk of a prefix wave: nk tiles from tile b0 of the row, every one for
// kPrefixSets sets of sixteen query columns (st[j] / qb[j]), so that one load
// of a tile serves 16 * kPrefixSets columns.  One tile is in registers: per
// tile the score MFMAs of all sets run first, then the K half is refilled
// with the next tile, the V half is repacked into the eight P V operands
// (once for all sets) and refilled, then each set's softmax and P V.  Every
// position of the prefix is below every length, so nothing is masked.  The
// walk is bound by its own instructions, not by the loads (one tile ahead
// measured as fast as two to four), so the registers a second tile would
// take hold the operands instead; the last refill repeats the last tile.
// The walk of each chunk of up to 64 tiles starts `rot` tiles into it and
// wraps around: the waves that read the same tiles for other columns start at
// other tiles.
__device__ __forceinline__ void prefix_walk(State (&st)[kPrefixSets], const bf16x8_t (&qb)[kPrefixSets][kKK],
                                            const int32_t* row, int nk, int b0, int rot, const WalkCtx& c) {
    Tile tt;
    auto tile_ptrs = [&](int tv0, int tv1, int e, int k, const uint4*& kt, const uint4*& vt) {
        uint32_t p0 = (uint32_t)__builtin_amdgcn_readlane(tv0, k);
        p0 = p0 < c.num_blocks ? p0 : c.num_blocks - 1;   // stay inside the pool whatever the table says
        if (c.pair8) {
            uint32_t p1 = (uint32_t)__builtin_amdgcn_readlane(tv1, k);
            p1 = p1 < c.num_blocks ? p1 : c.num_blocks - 1;
            kt = c.kpool + (size_t)(c.n < 8 ? p0 : p1) * c.block_stride + c.head_off;
            vt = c.vpool + (size_t)(c.r < 2 ? p0 : p1) * c.block_stride + c.head_off;
        } else {
            const size_t base = (size_t)p0 * c.block_stride + c.head_off +
                                (size_t)(e & ((1 << c.sub_shift) - 1)) * (kTileTokens * kRC);
            kt = c.kpool + base;
            vt = c.vpool + base;
        }
    };
    for (int k0 = 0; k0 < nk; k0 += 64) {
        const int nc = min(64, nk - k0);
        const int r0 = rot % nc;
        auto rk = [&](int k) { return k + r0 < nc ? k + r0 : k + r0 - nc; };   // step k (< nc) -> its tile
        const int2 tv = tile_entries(row, b0 + k0 + c.lane, c.lane < nc, c);
        const uint4 *kt, *vt;
        tile_ptrs(tv.x, tv.y, b0 + k0 + rk(0), rk(0), kt, vt);
        load_k(tt, kt, c.k_off);
        asm volatile("" : : : "memory");
        load_v(tt, vt, c.v_off, true);
        asm volatile("" : : : "memory");
        for (int k = 0; k < nc; ++k) {
            const int kn = rk(min(k + 1, nc - 1));
            tile_ptrs(tv.x, tv.y, b0 + k0 + kn, kn, kt, vt);
            __builtin_amdgcn_sched_barrier(0);
            f32x4_t sc[kPrefixSets];
#pragma unroll
            for (int j = 0; j < kPrefixSets; ++j) {
                sc[j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int kk = 0; kk < kKK; ++kk)
                    sc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, tt.k[kk]), qb[j][kk],
                                                                    sc[j], 0, 0, 0);
                asm volatile("" : "+v"(sc[j]) : : "memory");
            }
            load_k(tt, kt, c.k_off);
            // operand e: dim 8n + e of tokens 4r..4r+3, twice (P_hi and P_lo positions)
            bf16x8_t vop[8];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t x0 = (&tt.v[0].x)[w], x1 = (&tt.v[1].x)[w];
                const uint32_t x2 = (&tt.v[2].x)[w], x3 = (&tt.v[3].x)[w];
                const uint32_t e0 = (x0 & 0xFFFFu) | (x1 << 16), e1 = (x2 & 0xFFFFu) | (x3 << 16);
                const uint32_t o0 = (x0 >> 16) | (x1 & 0xFFFF0000u), o1 = (x2 >> 16) | (x3 & 0xFFFF0000u);
                vop[2 * w] = as_operand(e0, e1, e0, e1);
                vop[2 * w + 1] = as_operand(o0, o1, o0, o1);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) asm volatile("" : "+v"(vop[e]) : : "memory");
            load_v(tt, vt, c.v_off, true);
#pragma unroll
            for (int j = 0; j < kPrefixSets; ++j)
                softmax_pv_core<16>(st[j], sc[j], [&](int e) __attribute__((always_inline)) { return vop[e]; }, c.r,
                                    c.n, c.sl2, 1.0f);
        }
    }
}

// One prefix wave: (column group, KV head, part).  A column group is
// 16 * kPrefixSets query columns; column n of set j is query head n % G of
// sequence (group * kPrefixSets + j) * 16 / G + n / G (zero past the batch).
template <int G, bool kAnyB>
__device__ void prefix_wave(const DecodeArgs& a, int64_t idx) {
    constexpr int kSeqs = 16 / G;   // sequences per set of sixteen columns
    const int Hkv = a.num_kv_heads;
    const int groups = ((a.num_seqs * G + 15) / 16 + kPrefixSets - 1) / kPrefixSets;
    const int kv = (int)(idx % Hkv);
    const int qg = (int)((idx / Hkv) % groups);
    const int p = (int)(idx / ((int64_t)Hkv * groups));
    const int b0 = p * a.prefix_part_tiles;
    const int nk = min(a.prefix_part_tiles, a.shared_tiles - b0);   // >= 1: the host sizes the parts

    WalkCtx c = make_ctx<kAnyB, false>(a, kv);
    bf16x8_t qb_op[kPrefixSets][kKK];
    State st[kPrefixSets];
#pragma unroll
    for (int j = 0; j < kPrefixSets; ++j) {
        const int col_seq = (qg * kPrefixSets + j) * kSeqs + c.n / G;
        const bool col_ok = col_seq < a.num_seqs;
        const size_t col_row = (size_t)(col_ok ? col_seq : 0) * a.num_q_heads + (size_t)kv * G + c.n % G;
        const uint4* qrow = reinterpret_cast<const uint4*>(a.q) + col_row * kRC;
#pragma unroll
        for (int kk = 0; kk < kKK; ++kk) {
            uint4 x = make_uint4(0u, 0u, 0u, 0u);
            if (col_ok) x = qrow[kk * 4 + c.r];
            qb_op[j][kk] = __builtin_bit_cast(bf16x8_t, x);
        }
        init_state(st[j]);
    }
    // every sequence covers the whole prefix: no position is masked
    prefix_walk(st, qb_op, a.tables, nk, b0, qg, c);

    // lane (r, n): outputs of columns 4r .. 4r+3, dims 8n .. 8n+7; (m, l) of column n
    const int slots = a.prefix_parts + 1;
#pragma unroll
    for (int j = 0; j < kPrefixSets; ++j) {
        const float l_tot = total_l(st[j]);
        const int seq0 = (qg * kPrefixSets + j) * kSeqs;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int col = 4 * c.r + i;
            const int sq = seq0 + col / G;
            if (sq < a.num_seqs) {
                const size_t row = (size_t)sq * a.num_q_heads + (size_t)kv * G + col % G;
                float4* dst = reinterpret_cast<float4*>(a.ws_pacc + (row * slots + p) * kD + c.n * 8);
                dst[0] = make_float4(st[j].o[0][i], st[j].o[1][i], st[j].o[2][i], st[j].o[3][i]);
                dst[1] = make_float4(st[j].o[4][i], st[j].o[5][i], st[j].o[6][i], st[j].o[7][i]);
            }
        }
        const int sq = seq0 + c.n / G;
        if (c.r == 0 && sq < a.num_seqs) {
            const size_t row = (size_t)sq * a.num_q_heads + (size_t)kv * G + c.n % G;
            reinterpret_cast<float2*>(a.ws_pml)[row * slots + p] = make_float2(st[j].m, l_tot);
        }
    }
}

template <int G, bool kAnyB, bool kFp8>
__global__ __launch_bounds__(kWave) void decode_bf16_streamk_kernel(DecodeArgs a) {
    const int lane = threadIdx.x;
    const int64_t W = a.workers;
    const int64_t w = blockIdx.x;
    if (w >= W) {
        if constexpr (!kFp8) {
            if (a.shared_tiles > 0) {   // a shared prefix: its walks
                prefix_wave<G, kAnyB>(a, w - W);
                return;
            }
        }
        const int64_t x = w - W;
        if (x < a.append_waves) {   // decode append: the pool side
            if constexpr (!kFp8) append_scatter_waves(a, x, a.append_waves);   // FP8: the walk stores the rows
        } else {
            const int64_t nrow_waves = (int64_t)gridDim.x - W - a.append_waves;
            if constexpr (kFp8) fp8_rows_waves(a, x - a.append_waves, nrow_waves);
            else rows_scatter_waves(a, x - a.append_waves, nrow_waves);
        }
        return;
    }
    const int S = a.num_seqs;
    const int Hkv = a.num_kv_heads;

    // Tiles per sequence and their exclusive prefix sums, 64 sequences per
    // chunk: every lane loads the lengths of all chunks at once (one memory
    // round trip), then the chunks are scanned in registers.  Worker 0 also
    // records the prefix sums for the fix-up.
    constexpr int kMaxChunks = kStreamKMaxSeqs / kWave;
    const int nchunks = (S + kWave - 1) / kWave;
    int len_c[kMaxChunks];
    load_chunk_lens(a, S, nchunks, lane, len_c);
#pragma unroll
    for (int ch = 0; ch < kMaxChunks; ++ch) {
        const int L = clamp_len(len_c[ch], a.max_context) - a.shared_tiles * kTileTokens;   // walk_len
        len_c[ch] = (ch < nchunks && ch * kWave + lane < S && L > 0) ? L : 0;
    }
    // positions in 32 bits: the host takes this kernel only for batches of
    // fewer than kMaxSplitPositions
    int64_t ex_c[kMaxChunks];
    int T32 = 0;
#pragma unroll
    for (int ch = 0; ch < kMaxChunks; ++ch) {
        if (ch < nchunks) {
            const int nt = Hkv * (int)walk_span((len_c[ch] + kTileTokens - 1) / kTileTokens, a.piece_cost);
            const int incl = wave_inclusive_sum(nt);
            ex_c[ch] = T32 + incl - nt;
            if (w == 0 && ch * kWave + lane < S) a.ws_prefix[ch * kWave + lane] = ex_c[ch];
            T32 += __builtin_amdgcn_readlane(incl, kWave - 1);
        }
    }
    asm volatile("" : "+v"(T32));   // kept in a vector register, as the walk's other split values
    const int64_t T = T32;
    if (w == 0 && lane == 0) a.ws_prefix[S] = T;
    int64_t t = slice_start(w, T, a.split);
    const int64_t t_end = slice_start(w + 1, T, a.split);
    if (t >= t_end) return;

    // the sequence holding position t: the lane whose [excl, excl + positions) contains it
    int seq = S, L = 0;
    int64_t seq_first = 0;
#pragma unroll
    for (int ch = 0; ch < kMaxChunks; ++ch) {
        if (ch < nchunks && seq == S) {
            const int nt = Hkv * (int)walk_span((len_c[ch] + kTileTokens - 1) / kTileTokens, a.piece_cost);
            const uint64_t bal = __builtin_amdgcn_ballot_w64(nt > 0 && ex_c[ch] <= t && t < ex_c[ch] + nt);
            if (bal) {
                const int j = __builtin_ctzll(bal);
                seq = ch * kWave + j;
                seq_first = readlane64(ex_c[ch], j);
                L = __builtin_amdgcn_readlane(len_c[ch], j);
            }
        }
    }
    seq = __builtin_amdgcn_readfirstlane(seq);
    L = __builtin_amdgcn_readfirstlane(L);
    int nblk = (L + kTileTokens - 1) / kTileTokens;   // 16-token tiles
    // position t lies in the span of walk (seq, kv); t moves to the split
    // position of the first tile this slice walks there (past the span's
    // leading positions; at or past t_end when the slice ends among them)
    const int64_t off = t - seq_first;
    const int64_t span = walk_span(nblk, a.piece_cost);
    if (seq >= S || span <= 0) return;   // no sequence holds t: not reached with consistent lengths
    int kv = div_small(off, span);   // < Hkv: off < Hkv span <= T < 2^31
    if (kv >= Hkv) return;
    const int64_t at = off - (int64_t)kv * span;
    int b = first_tile_at(at, a.piece_cost);
    t += a.piece_cost + b - at;

    // The stores that end a piece: its output rows (a walk it covered whole),
    // its state after a shared prefix, or its split record.  A piece that
    // another piece of this slice follows is parked in LDS instead (Parked)
    // and stored when the slice ends.
    auto emit = [&](const State& so, float l_tot, int seq_, int kv_, bool whole_, bool first_)
        __attribute__((always_inline)) {
        const int r = lane >> 4, n = lane & 15;
        if (whole_ && a.shared_tiles > 0) {   // after a shared prefix: a state for the fix-up to merge
            const int slots = a.prefix_parts + 1;
            const size_t row0 = (size_t)seq_ * a.num_q_heads + (size_t)kv_ * G;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int h = 4 * r + j;
                if (h < G) {
                    float4* dst = reinterpret_cast<float4*>(a.ws_pacc + ((row0 + h) * slots + a.prefix_parts) * kD +
                                                            n * 8);
                    dst[0] = make_float4(so.o[0][j], so.o[1][j], so.o[2][j], so.o[3][j]);
                    dst[1] = make_float4(so.o[4][j], so.o[5][j], so.o[6][j], so.o[7][j]);
                }
            }
            if (r == 0 && n < G)
                reinterpret_cast<float2*>(a.ws_pml)[(row0 + n) * slots + a.prefix_parts] = make_float2(so.m, l_tot);
        } else if (whole_) {
            uint4* orow = reinterpret_cast<uint4*>(a.out) + ((size_t)seq_ * a.num_q_heads + (size_t)kv_ * G) * kRC;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int h = 4 * r + j;
                const float lh = __shfl(l_tot, h & 15, kWave);
                if (h < G) {
                    const float inv = lh > 0.0f ? 1.0f / lh : 0.0f;
                    uint4 o;
                    o.x = pack_bf16x2(so.o[0][j] * inv, so.o[1][j] * inv);
                    o.y = pack_bf16x2(so.o[2][j] * inv, so.o[3][j] * inv);
                    o.z = pack_bf16x2(so.o[4][j] * inv, so.o[5][j] * inv);
                    o.w = pack_bf16x2(so.o[6][j] * inv, so.o[7][j] * inv);
                    orow[h * kRC + n] = o;
                }
            }
        } else {
            float* rec = record_ptr<G>(a, 2 * w + (first_ ? 0 : 1));
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int h = 4 * r + j;
                if (h < G) {
                    float4* dst = reinterpret_cast<float4*>(rec + h * kD + n * 8);
                    dst[0] = make_float4(so.o[0][j], so.o[1][j], so.o[2][j], so.o[3][j]);
                    dst[1] = make_float4(so.o[4][j], so.o[5][j], so.o[6][j], so.o[7][j]);
                }
            }
            if (r == 0 && n < G) {
                rec[G * kD + 2 * n] = so.m;
                rec[G * kD + 2 * n + 1] = l_tot;
            }
        }
    };
    __shared__ Parked<G, kParkedPieces> parked;   // tag: (sequence, KV head, whole, first piece)
    int nparked = 0;

    bool first_piece = true;
    bool pf_valid = false;   // table entries of the next piece fetched ahead
    int pf_seq = -1, pf_tv0 = 0, pf_tv1 = 0, pf_nb = 0;
    // tiles in registers; `primed`: they hold the first tiles of the piece fetched ahead
    static_assert(kBalancedDepth == 1, "a next piece is only known to have one tile");
    typename TileOf<kFp8>::type tt[kBalancedDepth];
    bool primed = false;
    while (t < t_end && seq < S) {
        const int n_here = (int)min((int64_t)(nblk - b), t_end - t);
        const bool whole = (b == 0) && (n_here == nblk);

        WalkCtx c = make_ctx<kAnyB, kFp8>(a, kv);
        c.row_len = a.max_blocks - a.shared_entries;   // the walk's row starts after a shared prefix
        const bool use_pf = pf_valid && pf_seq == seq && b == 0;
        c.keep_v = use_pf ? keep_v_fetched<kFp8>(pf_tv0, pf_nb, seq, S) : keep_v_cached<kFp8>(a, seq, b, c);
        bf16x8_t qb[kKK];
        load_q<G, kFp8>(qb, a, seq, kv, c);
        State st;
        init_state(st);
        // the piece that ends with the sequence's last block takes the appended row
        AppendRow app;
        app.active = a.k_append != nullptr && b + n_here == nblk;
        app.store = kFp8;   // FP8: the pool side of the append is this walk (no append waves)
        app.tok0 = (nblk - 1) * kTileTokens;
        app.j = (L - 1) % kTileTokens;
        app.brow = (L - 1) & ((kAnyB ? a.block_size : kTileTokens) - 1);   // block sizes are powers of two
        app.opens = app.brow == 0;
        app.krow = reinterpret_cast<const uint4*>(a.k_append) + ((size_t)seq * Hkv + kv) * kRC;
        app.vrow = reinterpret_cast<const uint4*>(a.v_append) + ((size_t)seq * Hkv + kv) * kRC;
        // The next piece of this slice, if it starts a new (sequence, KV head),
        // begins at block 0 of (seq, kv + 1) or of the next sequence: fetch its
        // first table entries now, so that piece waits for its tiles only.
        const int tv0_here = pf_tv0, tv1_here = pf_tv1;
        pf_valid = false;
        NextWalk nxt = no_next_walk();
        if (b + n_here == nblk && t + n_here + a.piece_cost < t_end) {
            const int nseq = kv + 1 < Hkv ? seq : seq + 1;
            if (nseq < S) {
                // tiles 0..63 of the next sequence's row; a lane whose tile would
                // need an entry past the row loads nothing (the walk never reads it)
                const bool ok = tile_in_row(c.lane, c.row_len, c.pair8, c.sub_shift);
                const int2 pf = tile_entries(walk_row(a, nseq), c.lane, ok, c);
                pf_tv0 = pf.x;
                pf_tv1 = pf.y;
                pf_nb = neighbour_entries<kFp8>(a, nseq, 0, c);
                pf_seq = nseq;
                pf_valid = true;
                // its first tile is fetched by this walk's last refill (wasted if
                // nseq turns out to be empty: the piece after it is then another one)
                nxt.valid = true;
                nxt.tv0 = pf.x;
                nxt.tv1 = pf.y;
                nxt.e0 = 0;
                nxt.head_off = (size_t)(kv + 1 < Hkv ? kv + 1 : 0) * c.head_stride;
                nxt.count = 1;
            }
        }
        primed = walk<G, kBalancedDepth, kFp8>(st, tt, primed && use_pf, qb, walk_row(a, seq), 1, n_here, b, L, c,
                                               app, use_pf, tv0_here, tv1_here, nxt);
        const float l_tot = total_l(st);

        const bool more = t + n_here < t_end;   // another piece follows in this slice
        if (more && nparked < kParkedPieces) {
            parked.put(nparked++, st, l_tot, make_int4(seq, kv, whole ? 1 : 0, first_piece ? 1 : 0), lane);
        } else {
            emit(st, l_tot, seq, kv, whole, first_piece);
        }

        // next piece: the next walk's first tile is piece_cost positions on
        // (walks with no tiles take no positions)
        t += n_here;
        first_piece = false;
        b += n_here;
        if (b == nblk) {
            b = 0;
            if (++kv == Hkv) {
                kv = 0;
                do {
                    ++seq;
                    L = (seq < S) ? __builtin_amdgcn_readfirstlane(walk_len(a, seq)) : 0;
                    nblk = (L + kTileTokens - 1) / kTileTokens;
                } while (nblk == 0 && seq < S && t < t_end);
            }
            t += a.piece_cost;
        }
    }
    for (int i = 0; i < nparked; ++i) {
        State so;
        const int4 tag = parked.get(i, so, lane);
        emit(so, so.l, tag.x, tag.y, tag.z != 0, tag.w != 0);
    }
}

// ---------------------------------------------------------------------------
// Fixed partitions, persistent: the (sequence, KV head, partition) items of
// the whole batch, in that order, go to the same single-wave workers as the
// balanced split.  Worker w takes every item whose first tile lies in its
// tile slice [slice_start(w), slice_start(w + 1)) and walks it whole, so each
// partition's state comes from one wave, as the partition merge expects, and
// the workers' loads differ by at most one partition.  A one-workgroup-per-
// partition grid instead pays the latency of a table load and of the first
// tiles for every partition, and launches a workgroup for every slot of the
// (max partitions, KV heads, sequences) grid, most of them empty when lengths
// vary (70B-shaped batch: 874 us in that form).  Sequences of length 0 are
// written by the merge kernel.
// ---------------------------------------------------------------------------
template <int G, bool kAnyB, bool kFp8>
__global__ __launch_bounds__(kWave) void decode_partitions_kernel(DecodeArgs a) {
    const int lane = threadIdx.x;
    const int64_t W = gridDim.x;
    const int64_t w = blockIdx.x;
    const int S = a.num_seqs;
    const int Hkv = a.num_kv_heads;
    const int pt = a.part_tokens / kTileTokens;   // tiles per partition

    // tiles per sequence and their exclusive prefix sums, as in the balanced split
    constexpr int kMaxChunks = kStreamKMaxSeqs / kWave;
    const int nchunks = (S + kWave - 1) / kWave;
    int len_c[kMaxChunks];
    load_chunk_lens(a, S, nchunks, lane, len_c);
#pragma unroll
    for (int ch = 0; ch < kMaxChunks; ++ch)
        len_c[ch] = (ch < nchunks && ch * kWave + lane < S) ? clamp_len(len_c[ch], a.max_context) : 0;
    int64_t ex_c[kMaxChunks];
    int64_t T = 0;
#pragma unroll
    for (int ch = 0; ch < kMaxChunks; ++ch) {
        if (ch < nchunks) {
            const int64_t nt = (int64_t)Hkv * ((len_c[ch] + kTileTokens - 1) / kTileTokens);
            int64_t incl = nt;
#pragma unroll
            for (int off = 1; off < kWave; off <<= 1) {
                const int64_t y = __shfl_up(incl, off, kWave);
                if (lane >= off) incl += y;
            }
            ex_c[ch] = T + incl - nt;
            T += __shfl(incl, kWave - 1, kWave);
        }
    }
    const int64_t t_lo = slice_start(w, T, a.split);
    const int64_t t_hi = slice_start(w + 1, T, a.split);
    if (t_lo >= t_hi) return;

    int seq = S, L = 0;
    int64_t seq_first = 0;
#pragma unroll
    for (int ch = 0; ch < kMaxChunks; ++ch) {
        if (ch < nchunks && seq == S) {
            const int64_t nt = (int64_t)Hkv * ((len_c[ch] + kTileTokens - 1) / kTileTokens);
            const uint64_t bal = __builtin_amdgcn_ballot_w64(nt > 0 && ex_c[ch] <= t_lo && t_lo < ex_c[ch] + nt);
            if (bal) {
                const int j = __builtin_ctzll(bal);
                seq = ch * kWave + j;
                seq_first = readlane64(ex_c[ch], j);
                L = __builtin_amdgcn_readlane(len_c[ch], j);
            }
        }
    }
    seq = __builtin_amdgcn_readfirstlane(seq);
    L = __builtin_amdgcn_readfirstlane(L);
    int nblk = (L + kTileTokens - 1) / kTileTokens;
    const int64_t off = t_lo - seq_first;
    int kv = (int)(off / nblk);
    int b = (int)(off - (int64_t)kv * nblk);
    b = (b + pt - 1) / pt * pt;   // the first partition that starts in this slice

    // The stores that end a partition: the output rows (a context of one
    // partition) or its state for the merge; parked in LDS while another
    // partition of this slice follows (Parked).
    auto emit = [&](const State& so, float l_tot, int seq_, int kv_, int part_, bool whole_)
        __attribute__((always_inline)) {
        const int r = lane >> 4, n = lane & 15;
        if (whole_) {   // the whole context: the output itself
            uint4* orow = reinterpret_cast<uint4*>(a.out) + ((size_t)seq_ * a.num_q_heads + (size_t)kv_ * G) * kRC;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int h = 4 * r + j;
                const float lh = __shfl(l_tot, h & 15, kWave);
                if (h < G) {
                    const float inv = lh > 0.0f ? 1.0f / lh : 0.0f;
                    uint4 o;
                    o.x = pack_bf16x2(so.o[0][j] * inv, so.o[1][j] * inv);
                    o.y = pack_bf16x2(so.o[2][j] * inv, so.o[3][j] * inv);
                    o.z = pack_bf16x2(so.o[4][j] * inv, so.o[5][j] * inv);
                    o.w = pack_bf16x2(so.o[6][j] * inv, so.o[7][j] * inv);
                    orow[h * kRC + n] = o;
                }
            }
        } else {   // this partition's (m, l, unnormalised output) for the merge kernel
            const size_t row0 = (size_t)seq_ * a.num_q_heads + (size_t)kv_ * G;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int h = 4 * r + j;
                if (h < G) {
                    const size_t slot = (row0 + h) * a.max_parts + part_;
                    float4* dst = reinterpret_cast<float4*>(a.ws_acc + slot * kD + n * 8);
                    dst[0] = make_float4(so.o[0][j], so.o[1][j], so.o[2][j], so.o[3][j]);
                    dst[1] = make_float4(so.o[4][j], so.o[5][j], so.o[6][j], so.o[7][j]);
                }
            }
            if (r == 0 && n < G)
                reinterpret_cast<float2*>(a.ws_ml)[(row0 + n) * a.max_parts + part_] = make_float2(so.m, l_tot);
        }
    };
    constexpr int kParked = parked_partitions<G>();
    __shared__ Parked<G, kParked> parked;   // tag: (sequence, KV head, partition, whole context)
    int nparked = 0;

    AppendRow none;
    none.active = false;
    none.store = false;
    none.opens = false;
    none.brow = 0;
    none.krow = none.vrow = nullptr;
    bool pf_valid = false;   // table entries of the next partition fetched ahead
    int pf_kv = -1, pf_b = -1, pf_tv0 = 0, pf_tv1 = 0, pf_nb = 0;
    // tiles in registers; `primed`: they hold the first tiles of the partition fetched ahead
    typename TileOf<kFp8>::type tt[kPartitionDepth];
    bool primed = false;
    while (seq < S) {
        if (b >= nblk) {   // past this (sequence, KV head): the next one with tiles
            b = 0;
            if (++kv == Hkv) {
                kv = 0;
                do {
                    seq_first += (int64_t)Hkv * nblk;
                    ++seq;
                    L = (seq < S) ? __builtin_amdgcn_readfirstlane(clamp_len(a.lens[seq], a.max_context)) : 0;
                    nblk = (L + kTileTokens - 1) / kTileTokens;
                } while (nblk == 0 && seq < S);
                if (seq >= S) break;
            }
            continue;
        }
        if (seq_first + (int64_t)kv * nblk + b >= t_hi) break;   // the next worker's partition
        const int n_here = min(pt, nblk - b);
        const int part = b / pt;
        const int nparts = (L + a.part_tokens - 1) / a.part_tokens;

        WalkCtx c = make_ctx<kAnyB, kFp8>(a, kv);
        const bool use_pf = pf_valid && pf_kv == kv && pf_b == b;   // pf_valid only within one sequence
        const int tv0_here = pf_tv0, tv1_here = pf_tv1;
        c.keep_v = use_pf ? keep_v_fetched<kFp8>(pf_tv0, pf_nb, seq, S) : keep_v_cached<kFp8>(a, seq, b, c);
        // The next partition, when it lies in this sequence and in this slice:
        // fetch its first table entries now, so that it waits for its tiles only.
        pf_valid = false;
        NextWalk nxt = no_next_walk();
        {
            int nb = b + pt, nkv = kv;
            if (nb >= nblk) {
                nb = 0;
                ++nkv;
            }
            if (nkv < Hkv && seq_first + (int64_t)nkv * nblk + nb < t_hi) {
                const int e = nb + c.lane;
                const bool ok = tile_in_row(e, c.row_len, c.pair8, c.sub_shift);
                const int2 pf = tile_entries(a.tables + (size_t)seq * a.max_blocks, e, ok, c);
                pf_tv0 = pf.x;
                pf_tv1 = pf.y;
                pf_nb = neighbour_entries<kFp8>(a, seq, nb, c);
                pf_kv = nkv;
                pf_b = nb;
                pf_valid = true;
                // its first tiles are fetched by this walk's last refills
                nxt.valid = true;
                nxt.tv0 = pf.x;
                nxt.tv1 = pf.y;
                nxt.e0 = nb;
                nxt.head_off = (size_t)nkv * c.head_stride;
                nxt.count = min(64, min(pt, nblk - nb));   // its first chunk
            }
        }
        bf16x8_t qb[kKK];
        load_q<G, kFp8>(qb, a, seq, kv, c);
        State st;
        init_state(st);
        primed = walk<G, kPartitionDepth, kFp8>(st, tt, primed && use_pf, qb, a.tables + (size_t)seq * a.max_blocks,
                                                1, n_here, b, L, c, none, use_pf, tv0_here, tv1_here, nxt);
        const float l_tot = total_l(st);
        // another partition of this slice follows (the next one starts here)
        const bool more = seq_first + (int64_t)kv * nblk + min(b + pt, nblk) < t_hi;
        if (more && nparked < kParked)
            parked.put(nparked++, st, l_tot, make_int4(seq, kv, part, nparts == 1 ? 1 : 0), lane);
        else
            emit(st, l_tot, seq, kv, part, nparts == 1);
        b += pt;
    }
    for (int i = 0; i < nparked; ++i) {
        State so;
        const int4 tag = parked.get(i, so, lane);
        emit(so, so.l, tag.x, tag.y, tag.z, tag.w != 0);
    }
}


// Fix-up for one (sequence, KV head): zeros for an empty sequence; nothing if
// one slice held it whole; otherwise the log-sum-exp merge of the partial
// states its slices left.  With fewer tiles than workers some slices are
// empty; they left nothing and are skipped.
//
// One wave per GH of the G query heads: lanes first read the (m, l) pairs of
// up to 64 records at once and reduce them across the wave; then each lane
// sums two dims of each of its heads over the records, several records'
// loads in flight at a time.  Splitting a pair's heads over G / GH waves
// shortens each wave's chain of dependent steps when there are few pairs
// (see launch_streamk_fixup).
template <int G, int GH>
__global__ __launch_bounds__(kWave) void streamk_fixup_kernel(DecodeArgs a, int num_workers) {
    static_assert(G % GH == 0, "a wave takes GH of the group's G heads");
    const int kv = blockIdx.x / (G / GH);
    const int h0 = (blockIdx.x % (G / GH)) * GH;   // the wave's first head within the group
    const int seq = blockIdx.y;
    const int lane = threadIdx.x;
    // the length and the two prefix sums are independent: one memory round trip for all three
    const int L_all = clamp_len(a.lens[seq], a.max_context);
    const int64_t T = a.ws_prefix[a.num_seqs];
    const int64_t first_tile = a.ws_prefix[seq];
    uint32_t* out =
        reinterpret_cast<uint32_t*>(a.out) + ((size_t)seq * a.num_q_heads + (size_t)kv * G + h0) * (kD / 2);
    if (L_all == 0) {
#pragma unroll
        for (int h = 0; h < GH; ++h) out[h * (kD / 2) + lane] = 0u;
        return;
    }
    // with a shared prefix the balanced walk covered only the tokens after it
    const bool shared = a.shared_tiles > 0;
    const int L = shared ? (L_all > a.shared_tiles * kTileTokens ? L_all - a.shared_tiles * kTileTokens : 0) : L_all;
    const int nblk = (L + kTileTokens - 1) / kTileTokens;   // 16-token tiles
    const int64_t W = num_workers;
    const int64_t base = first_tile + (int64_t)kv * walk_span(nblk, a.piece_cost);   // the walk's positions start here
    const int64_t s0 = base + a.piece_cost;                                            // ... and its tile 0 sits here
    const double rcp_T = nblk > 0 ? 1.0 / (double)T : 0.0;
    const int64_t w0 = nblk > 0 ? worker_of(s0, T, rcp_T, a.split) : 0;
    const int64_t w1 = nblk > 0 ? worker_of(s0 + nblk - 1, T, rcp_T, a.split) : 0;
    if (w0 == w1 && !shared) return;   // written by its worker
    // records of the slices that split the walk (none when one slice held it whole)
    const int nrec = (nblk > 0 && w0 != w1) ? (int)(w1 - w0 + 1) : 0;

    // record slot of worker w0 + j, or -1 for an empty slice.  Worker w0 left
    // its second record when its slice began before this walk's span (the
    // positions just before the span are the last tiles of an earlier walk,
    // which it walked first), else its first.
    auto slot_of = [&](int j) -> int64_t {
        const int64_t w = w0 + j;
        const int64_t st = slice_start(w, T, a.split);
        if (slice_start(w + 1, T, a.split) <= st) return -1;
        return (w == w0 && st < base) ? 2 * w + 1 : 2 * w;
    };

    // Records are taken 64 at a time, lane j holding the (m, l) pairs of record
    // j0 + j.  Per block of records: the block's max of each head (a wave
    // reduction), each lane's weight 2^(m_j - M) and the denominator (a wave
    // sum); every lane then sums two dims of every head over the records in
    // order, kU records' loads in flight at a time, and stops after the last
    // record (a wave-uniform test: most pairs have two or three records).
    constexpr int kU = GH >= 8 ? 4 : 8;   // eight heads a wave: 4 records' outputs, so the wave stays within 256 VGPRs
    float M[GH], den[GH], n0[GH], n1[GH];
#pragma unroll
    for (int h = 0; h < GH; ++h) {
        M[h] = -INFINITY;
        den[h] = n0[h] = n1[h] = 0.0f;
    }
    const int d = lane * 2;
    // The first 64 records' (m, l) pairs and the first kU records' partial
    // outputs are loaded before anything is merged: with a shared prefix their
    // round trip overlaps the prefix states' one.
    int cnt = min(kWave, nrec);
    int64_t slot = lane < cnt ? slot_of(lane) : -1;
    float m_j[GH], l_j[GH], f_j[GH];
    float2 x[kU][GH];
    auto load_ml = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < GH; ++h) {
            m_j[h] = -INFINITY;
            l_j[h] = 0.0f;
        }
        if (slot >= 0) {
            const float* ml = record_ptr<G>(a, slot) + G * kD + 2 * h0;
#pragma unroll
            for (int h = 0; h < GH; ++h) {
                m_j[h] = ml[2 * h];
                l_j[h] = ml[2 * h + 1];
            }
        }
    };
    auto load_x = [&](int jj) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t sl = readlane64(slot, min(jj + u, cnt - 1));
            const bool live = jj + u < cnt && sl >= 0;   // wave-uniform
            const float* rec = record_ptr<G>(a, live ? sl : 0) + h0 * kD;
#pragma unroll
            for (int h = 0; h < GH; ++h)
                x[u][h] = live ? *reinterpret_cast<const float2*>(rec + h * kD + d) : make_float2(0.0f, 0.0f);
        }
    };
    if (nrec > 0) {
        load_ml();
        load_x(0);
    }
    if (shared) {
        // the prefix parts, then (when one slice held the rest whole) its state,
        // in slot order; each lane two dims of each of its heads
        const int slots = a.prefix_parts + 1;
        const int nslot = a.prefix_parts + (nblk > 0 && w0 == w1 ? 1 : 0);
        const size_t row0 = (size_t)seq * a.num_q_heads + (size_t)kv * G + h0;
        constexpr int kUP = 32 / GH;   // slots in flight per batch (128 registers of loads)
        for (int p0 = 0; p0 < nslot; p0 += kUP) {
            float2 pml[kUP][GH], px[kUP][GH];
#pragma unroll
            for (int u = 0; u < kUP; ++u) {
                const bool live = p0 + u < nslot;   // wave-uniform
#pragma unroll
                for (int h = 0; h < GH; ++h) {
                    const size_t ps = (row0 + h) * slots + (live ? p0 + u : 0);
                    pml[u][h] = live ? reinterpret_cast<const float2*>(a.ws_pml)[ps] : make_float2(-INFINITY, 0.0f);
                    px[u][h] = live ? *reinterpret_cast<const float2*>(a.ws_pacc + ps * kD + d)
                                    : make_float2(0.0f, 0.0f);
                }
            }
#pragma unroll
            for (int h = 0; h < GH; ++h) {
                float mb = M[h];
#pragma unroll
                for (int u = 0; u < kUP; ++u) mb = fmaxf(mb, pml[u][h].x);
                const float corr = fast_exp2(M[h] - safe_ref(mb));   // 0 for the first batch
                n0[h] *= corr;
                n1[h] *= corr;
                den[h] *= corr;
                M[h] = mb;
#pragma unroll
                for (int u = 0; u < kUP; ++u) {
                    const float f = fast_exp2(pml[u][h].x - safe_ref(mb));   // 0 for an absent slot
                    den[h] = fmaf(pml[u][h].y, f, den[h]);
                    n0[h] = fmaf(px[u][h].x, f, n0[h]);
                    n1[h] = fmaf(px[u][h].y, f, n1[h]);
                }
            }
        }
    }
    for (int j0 = 0; j0 < nrec; j0 += kWave) {
        if (j0 > 0) {   // the next 64 records (the first block's loads were issued above)
            cnt = min(kWave, nrec - j0);
            slot = lane < cnt ? slot_of(j0 + lane) : -1;
            load_ml();
        }
        for (int jj = 0; jj < cnt; jj += kU) {
            if (j0 > 0 || jj > 0) load_x(jj);
            if (jj == 0) {   // the block's weights, while the first loads are in flight
#pragma unroll
                for (int h = 0; h < GH; ++h) {
                    const float m_new = fmaxf(M[h], wave_max(m_j[h]));
                    const float corr = fast_exp2(M[h] - safe_ref(m_new));   // 0 for the first block
                    n0[h] *= corr;
                    n1[h] *= corr;
                    den[h] *= corr;
                    M[h] = m_new;
                    f_j[h] = slot >= 0 ? fast_exp2(m_j[h] - safe_ref(m_new)) : 0.0f;
                    float w = l_j[h] * f_j[h];
#pragma unroll
                    for (int off = kWave / 2; off > 0; off >>= 1) w += __shfl_xor(w, off, kWave);
                    den[h] += w;
                }
            }
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                if (jj + u < cnt) {   // wave-uniform
#pragma unroll
                    for (int h = 0; h < GH; ++h) {
                        const float f = readlane_f(f_j[h], jj + u);
                        n0[h] = fmaf(x[u][h].x, f, n0[h]);
                        n1[h] = fmaf(x[u][h].y, f, n1[h]);
                    }
                }
            }
        }
    }
#pragma unroll
    for (int h = 0; h < GH; ++h) {
        const float inv = den[h] > 0.0f ? 1.0f / den[h] : 0.0f;
        out[h * (kD / 2) + lane] = pack_bf16x2(n0[h] * inv, n1[h] * inv);
    }
}

// The any-block-size instantiation: it holds the most registers of the
// kernels a pool type can launch, so its occupancy bounds them all.
template <int G, bool kFp8>
const void* streamk_kernel_ptr() {
    return reinterpret_cast<const void*>(&decode_bf16_streamk_kernel<G, true, kFp8>);
}

}  // namespace

int streamk_workers(int group, bool fp8) {
    // bf16 tiles: one worker wave per SIMD (four per compute unit).  With two
    // resident waves per SIMD the older one wins the SIMD's issue arbitration:
    // equal slices then finish about 1.5x apart, and the second half of the
    // kernel runs with one wave per SIMD anyway.  One wave per SIMD keeps all
    // workers at the same pace (timed per worker with the chip's realtime
    // counter) and is 4 % faster end to end on the 8B and 70B shapes.
    // FP8 tiles carry half the bytes for the same arithmetic, so a wave's
    // compute is a larger share of its time; a second wave per SIMD hides it
    // (8B shape: call 60.9 -> 60.3 us warm, 74.8 -> 69.8 us cold; 70B shape:
    // 201 -> 188 us).
    constexpr int kMaxDev = 16;
    const int waves_per_cu = fp8 ? 8 : 4;
    // per (device, pool type, group); several host threads may fill it at once with the same value
    static std::atomic<int> cached[kMaxDev][2][9];
    if (group < 1 || group > 8) return 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) {
        (void)hipGetLastError();
        return kStreamKDefaultWorkers;
    }
    const int known = cached[dev][fp8][group].load(std::memory_order_relaxed);
    if (known) return known;
    int cus = 0, per_cu = 0;
    const void* fn = nullptr;
    switch (group) {
        case 1: fn = fp8 ? streamk_kernel_ptr<1, true>() : streamk_kernel_ptr<1, false>(); break;
        case 2: fn = fp8 ? streamk_kernel_ptr<2, true>() : streamk_kernel_ptr<2, false>(); break;
        case 4: fn = fp8 ? streamk_kernel_ptr<4, true>() : streamk_kernel_ptr<4, false>(); break;
        case 8: fn = fp8 ? streamk_kernel_ptr<8, true>() : streamk_kernel_ptr<8, false>(); break;
        default: return 0;
    }
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kWave, 0) != hipSuccess || cus <= 0 || per_cu <= 0) {
        (void)hipGetLastError();
        return kStreamKDefaultWorkers;
    }
    const int workers = min(cus * min(per_cu, waves_per_cu), kMaxSplitWorkers);
    cached[dev][fp8][group].store(workers, std::memory_order_relaxed);
    return workers;
}

namespace {

// The balanced walk (a.workers and the slice weights already set).
template <bool kFp8>
hipError_t launch_streamk_walk(const DecodeArgs& a_in, int group, int workers, hipStream_t stream) {
    DecodeArgs a = a_in;
    // decode append: a few extra single-wave workgroups store the new rows
    // (bf16: about 8 chunks per lane; FP8: about 4 rows per wave)
    int64_t extra = 0;
    a.append_waves = 0;
    if (a.shared_tiles > 0) {   // the prefix walks: (column group, KV head, part)
        extra = prefix_column_groups(a.num_seqs, group) * a.num_kv_heads * a.prefix_parts;
    } else {
        if (a.k_append && !kFp8) {
            // bf16: beside the workers from the start.  FP8 pools: the walk that
            // takes a (sequence, KV head)'s last tile stores the row (AppendRow::store);
            // waves past the workers would only run at the launch's tail, once FP8
            // workers free their wave slots (8B-shaped step 71.0 us with them)
            const int64_t items = (int64_t)a.num_seqs * 2 * a.num_kv_heads * kRC;
            const int64_t per_wave = 8 * kWave;
            const int64_t cap = 256;
            extra = (items + per_wave - 1) / per_wave;
            extra = extra < 1 ? 1 : (extra > cap ? cap : extra);
            a.append_waves = (int32_t)extra;
        }
        // other rows: up to 768 waves (a row or a few each), so that they are
        // done while the workers still scan lengths and fetch their first
        // tiles; with 256 waves (nine rows each on the 70B-shaped step) the
        // step took 2 us longer.  FP8 pools: one (16-token chunk, KV head) item a wave.
        if (a.num_rows > 0) {
            const int64_t items = kFp8 ? (a.num_rows + 15) / 16 * a.num_kv_heads : a.num_rows;
            const int64_t cap = kFp8 ? 1024 : 768;
            extra += items < cap ? items : cap;
        }
    }
    dim3 grid((unsigned)(workers + extra));
    const bool any_b = a.block_size != kTileTokens;
    switch (group) {
        case 1:
            if (any_b) decode_bf16_streamk_kernel<1, true, kFp8><<<grid, kWave, 0, stream>>>(a);
            else decode_bf16_streamk_kernel<1, false, kFp8><<<grid, kWave, 0, stream>>>(a);
            break;
        case 2:
            if (any_b) decode_bf16_streamk_kernel<2, true, kFp8><<<grid, kWave, 0, stream>>>(a);
            else decode_bf16_streamk_kernel<2, false, kFp8><<<grid, kWave, 0, stream>>>(a);
            break;
        case 4:
            if (any_b) decode_bf16_streamk_kernel<4, true, kFp8><<<grid, kWave, 0, stream>>>(a);
            else decode_bf16_streamk_kernel<4, false, kFp8><<<grid, kWave, 0, stream>>>(a);
            break;
        case 8:
            if (any_b) decode_bf16_streamk_kernel<8, true, kFp8><<<grid, kWave, 0, stream>>>(a);
            else decode_bf16_streamk_kernel<8, false, kFp8><<<grid, kWave, 0, stream>>>(a);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// The fix-up after the walk: merges the records of (sequence, KV head) pairs
// split between workers (and, with a shared prefix, the prefix states).
hipError_t launch_streamk_fixup(const DecodeArgs& a, int group, int workers, hipStream_t stream) {
    // GH query heads per wave: the pair's heads go to several waves while
    // the grid would hold fewer than kFixupMinWaves (measured, same box:
    // 70B TP-8 shard, 256 pairs of 8 heads, 54.0 -> 49.5 us per call with two
    // heads per wave; 8B shape 103.2 -> 102.5 us; batches of 1024 pairs or
    // more run slower split: 70B shape 274 -> 275 us, prefix sharing 45.4 ->
    // 46.3 us)
    const int64_t pairs = (int64_t)a.num_seqs * a.num_kv_heads;
    int gh = group;
    while (gh > 1 && pairs * (group / gh) < kFixupMinWaves) gh /= 2;
    const dim3 grid((unsigned)(a.num_kv_heads * (group / gh)), (unsigned)a.num_seqs);
    switch (group * 16 + gh) {
        case 1 * 16 + 1: streamk_fixup_kernel<1, 1><<<grid, kWave, 0, stream>>>(a, workers); break;
        case 2 * 16 + 1: streamk_fixup_kernel<2, 1><<<grid, kWave, 0, stream>>>(a, workers); break;
        case 2 * 16 + 2: streamk_fixup_kernel<2, 2><<<grid, kWave, 0, stream>>>(a, workers); break;
        case 4 * 16 + 1: streamk_fixup_kernel<4, 1><<<grid, kWave, 0, stream>>>(a, workers); break;
        case 4 * 16 + 2: streamk_fixup_kernel<4, 2><<<grid, kWave, 0, stream>>>(a, workers); break;
        case 4 * 16 + 4: streamk_fixup_kernel<4, 4><<<grid, kWave, 0, stream>>>(a, workers); break;
        case 8 * 16 + 1: streamk_fixup_kernel<8, 1><<<grid, kWave, 0, stream>>>(a, workers); break;
        case 8 * 16 + 2: streamk_fixup_kernel<8, 2><<<grid, kWave, 0, stream>>>(a, workers); break;
        case 8 * 16 + 4: streamk_fixup_kernel<8, 4><<<grid, kWave, 0, stream>>>(a, workers); break;
        case 8 * 16 + 8: streamk_fixup_kernel<8, 8><<<grid, kWave, 0, stream>>>(a, workers); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <bool kFp8>
hipError_t launch_streamk(const DecodeArgs& a_in, int group, int workers, hipStream_t stream) {
    DecodeArgs a = a_in;
    a.workers = workers;
    a.split = split_consts(workers, kFp8 ? kFp8SliceWeights : kBf16SliceWeights);
    a.piece_cost = kFp8 ? kFp8PieceCost : kBf16PieceCost;
    hipError_t e = launch_streamk_walk<kFp8>(a, group, workers, stream);
    if (e != hipSuccess) return e;
    return launch_streamk_fixup(a, group, workers, stream);
}

template <bool kFp8>
hipError_t launch_partitions(const DecodeArgs& a_in, int group, int workers, hipStream_t stream) {
    DecodeArgs a = a_in;
    a.split = split_consts(workers, kFp8 ? kFp8SliceWeights : kBf16SliceWeights);
    dim3 grid((unsigned)workers);
    const bool any_b = a.block_size != kTileTokens;
    switch (group) {
        case 1:
            if (any_b) decode_partitions_kernel<1, true, kFp8><<<grid, kWave, 0, stream>>>(a);
            else decode_partitions_kernel<1, false, kFp8><<<grid, kWave, 0, stream>>>(a);
            break;
        case 2:
            if (any_b) decode_partitions_kernel<2, true, kFp8><<<grid, kWave, 0, stream>>>(a);
            else decode_partitions_kernel<2, false, kFp8><<<grid, kWave, 0, stream>>>(a);
            break;
        case 4:
            if (any_b) decode_partitions_kernel<4, true, kFp8><<<grid, kWave, 0, stream>>>(a);
            else decode_partitions_kernel<4, false, kFp8><<<grid, kWave, 0, stream>>>(a);
            break;
        case 8:
            if (any_b) decode_partitions_kernel<8, true, kFp8><<<grid, kWave, 0, stream>>>(a);
            else decode_partitions_kernel<8, false, kFp8><<<grid, kWave, 0, stream>>>(a);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <bool kFp8>
hipError_t launch_mfma(const DecodeArgs& a, int group, hipStream_t stream) {
    dim3 grid((unsigned)a.max_parts, (unsigned)a.num_kv_heads, (unsigned)a.num_seqs);
    dim3 block(kWaves * kWave);
    const bool any_b = a.block_size != kTileTokens;
    switch (group) {
        case 1:
            if (any_b) decode_bf16_mfma_kernel<1, true, kFp8><<<grid, block, 0, stream>>>(a);
            else decode_bf16_mfma_kernel<1, false, kFp8><<<grid, block, 0, stream>>>(a);
            break;
        case 2:
            if (any_b) decode_bf16_mfma_kernel<2, true, kFp8><<<grid, block, 0, stream>>>(a);
            else decode_bf16_mfma_kernel<2, false, kFp8><<<grid, block, 0, stream>>>(a);
            break;
        case 4:
            if (any_b) decode_bf16_mfma_kernel<4, true, kFp8><<<grid, block, 0, stream>>>(a);
            else decode_bf16_mfma_kernel<4, false, kFp8><<<grid, block, 0, stream>>>(a);
            break;
        case 8:
            if (any_b) decode_bf16_mfma_kernel<8, true, kFp8><<<grid, block, 0, stream>>>(a);
            else decode_bf16_mfma_kernel<8, false, kFp8><<<grid, block, 0, stream>>>(a);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_bf16_shared(const DecodeArgs& a, int group, int workers, hipStream_t stream) {
    if (a.shared_tiles <= 0 || a.prefix_parts <= 0 || a.prefix_part_tiles <= 0 ||
        a.shared_entries != (int32_t)((int64_t)a.shared_tiles * kTileTokens / a.block_size) ||
        (int64_t)(a.prefix_parts - 1) * a.prefix_part_tiles >= a.shared_tiles || !a.ws_pml || !a.ws_pacc || a.k_append)
        return hipErrorInvalidValue;
    if (group != 1 && group != 2 && group != 4 && group != 8) return hipErrorInvalidValue;
    return launch_streamk<false>(a, group, workers, stream);   // the prefix walks run as extra waves
}

hipError_t launch_decode_bf16_streamk(const DecodeArgs& a, int group, int workers, hipStream_t stream) {
    return launch_streamk<false>(a, group, workers, stream);
}

hipError_t launch_decode_fp8_streamk(const DecodeArgs& a, int group, int workers, hipStream_t stream) {
    return launch_streamk<true>(a, group, workers, stream);
}

hipError_t launch_decode_bf16_mfma(const DecodeArgs& a, int group, hipStream_t stream) {
    return launch_mfma<false>(a, group, stream);
}

hipError_t launch_decode_fp8_mfma(const DecodeArgs& a, int group, hipStream_t stream) {
    return launch_mfma<true>(a, group, stream);
}

hipError_t launch_decode_bf16_partitions(const DecodeArgs& a, int group, int workers, hipStream_t stream) {
    return launch_partitions<false>(a, group, workers, stream);
}

hipError_t launch_decode_fp8_partitions(const DecodeArgs& a, int group, int workers, hipStream_t stream) {
    return launch_partitions<true>(a, group, workers, stream);
}

}  // namespace kvp
