// Paged decode attention and the partition merge.
//
// What is computed (aicassindra.com "GPU paged KV cache", "Inside the paged
// attention kernel"; "PagedAttention, Internals First", "02 Block tables"):
// one workgroup per (sequence, KV head[, partition]) walks the sequence's
// logical blocks, reads each block's physical index from the block table,
// loads that block's K tile, forms the q.k scores of every query head in the
// KV head's group, folds them into a running online-softmax state and
// accumulates the V tile weighted by the softmax numerators.  Long contexts are
// cut into partitions handled by separate workgroups; a second kernel merges
// the partial (max, sum, output) states with a log-sum-exp rescale.
//
// Mapping onto a gfx950 compute unit (wave64):
//   * A (block, KV head) tile is block_size x head_dim contiguous elements
//     (4 KiB for bf16/D=128 and fp32/D=64).  One wave reads it with 16-byte
//     loads, each load instruction covering 1 KiB of consecutive bytes: lane l
//     takes token row i*TPL + l/LPT and the l%LPT-th 16-byte chunk of it.
//   * The q.k dot product of a token is split over the LPT lanes of its row
//     (bf16: packed dot2 instructions with fp32 accumulation) and summed with a
//     DPP butterfly inside the row, so every lane of the row holds the score.
//   * Online softmax state is kept per token row of each wave (each row sees
//     a fixed subset of token positions), so the block loop needs no
//     cross-row traffic; rows are merged by shuffles, and the waves of the
//     workgroup through LDS, once, at the end.
//   * The walk order depends only on logical positions, so the result is
//     bitwise independent of where blocks live in the pool.
#include <math.h>

#include "device_common.hpp"
#include "launch.hpp"

namespace kvp {

namespace {

constexpr int kDecodeWaves = 4;

template <int DT, int D>
struct Geo {
    static constexpr int kElemBytes = DT == 0 ? 4 : 2;
    static constexpr int kEpv = 16 / kElemBytes;            // elements per 16-byte lane load
    static constexpr int kRowChunks = D / kEpv;              // 16-byte chunks per token row (= lanes per row)
    static constexpr int kLpt = kRowChunks;
    static constexpr int kTpl = kWave / kLpt;                // token rows covered by one wave load
    static constexpr int kLoads = kBlockTokens / kTpl;       // wave loads per tile
    static_assert(kLpt * kTpl == kWave && kTpl * kLoads == kBlockTokens, "tile does not map onto a wave");
};

// Dot product of this lane's 16-byte chunks of q and k (fp32 accumulation).
template <int DT>
__device__ __forceinline__ float chunk_dot(const uint4& q, const uint4& k) {
    if constexpr (DT == 1) {
        float s = dot2_bf16(q.x, k.x, 0.0f);
        s = dot2_bf16(q.y, k.y, s);
        s = dot2_bf16(q.z, k.z, s);
        return dot2_bf16(q.w, k.w, s);
    } else {
        float s = __uint_as_float(q.x) * __uint_as_float(k.x);
        s = fmaf(__uint_as_float(q.y), __uint_as_float(k.y), s);
        s = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), s);
        return fmaf(__uint_as_float(q.w), __uint_as_float(k.w), s);
    }
}

// Widen a 16-byte chunk to fp32.
template <int DT>
__device__ __forceinline__ void chunk_to_f32(const uint4& v, float* f) {
    if constexpr (DT == 1) {
        f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
        f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
        f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
        f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
    } else {
        f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
        f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
    }
}

__device__ __forceinline__ float safe_max(float m) { return m == -INFINITY ? 0.0f : m; }

template <int DT, int D, int G>
__global__ __launch_bounds__(kDecodeWaves * kWave) void decode_kernel(DecodeArgs a) {
    using Gm = Geo<DT, D>;
    constexpr int EPV = Gm::kEpv, LPT = Gm::kLpt, TPL = Gm::kTpl, LOADS = Gm::kLoads;
    constexpr int RC = Gm::kRowChunks;

    const int part = blockIdx.x;
    const int kv = blockIdx.y;
    const int seq = blockIdx.z;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int r = lane / LPT;   // token row within a wave load
    const int c = lane % LPT;   // 16-byte chunk within the row

    int L = a.lens[seq];
    L = L < 0 ? 0 : (L > a.max_context ? a.max_context : L);
    const int nparts = L == 0 ? 1 : (L + a.part_tokens - 1) / a.part_tokens;
    if (part >= nparts) return;
    const int nblk = (L + kBlockTokens - 1) / kBlockTokens;
    const int bpp = a.part_tokens / kBlockTokens;
    const int b_begin = part * bpp;
    const int b_end = min(nblk, b_begin + bpp);

    // this lane's chunk of q for every query head of the group
    uint4 qv[G];
    {
        const uint4* qrow = reinterpret_cast<const uint4*>(a.q) + ((size_t)seq * a.num_q_heads + (size_t)kv * G) * RC;
#pragma unroll
        for (int h = 0; h < G; ++h) qv[h] = qrow[h * RC + c];
    }

    float m[G], l[G], acc[G][EPV];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.0f;
#pragma unroll
        for (int e = 0; e < EPV; ++e) acc[h][e] = 0.0f;
    }

    const int32_t* trow = a.tables + (size_t)seq * a.max_blocks;
    const uint4* kpool = reinterpret_cast<const uint4*>(a.k_layer);
    const uint4* vpool = reinterpret_cast<const uint4*>(a.v_layer);
    const float sl2 = a.scale_log2;

    for (int b = b_begin + wave; b < b_end; b += kDecodeWaves) {
        uint32_t phys = (uint32_t)trow[b];
        if (phys >= (uint32_t)a.num_blocks) phys = (uint32_t)a.num_blocks - 1;   // stay inside the pool
        const size_t tile = ((size_t)phys * a.num_kv_heads + kv) * (kBlockTokens * RC);
        uint4 kr[LOADS], vr[LOADS];
#pragma unroll
        for (int i = 0; i < LOADS; ++i) kr[i] = kpool[tile + (size_t)(i * TPL + r) * RC + c];
#pragma unroll
        for (int i = 0; i < LOADS; ++i) vr[i] = vpool[tile + (size_t)(i * TPL + r) * RC + c];

        float s[LOADS][G];
#pragma unroll
        for (int i = 0; i < LOADS; ++i)
#pragma unroll
            for (int h = 0; h < G; ++h) s[i][h] = group_sum<LPT>(chunk_dot<DT>(qv[h], kr[i])) * sl2;

        if ((b + 1) * kBlockTokens > L) {   // last, partially filled block: mask positions >= L
#pragma unroll
            for (int i = 0; i < LOADS; ++i) {
                if (b * kBlockTokens + i * TPL + r >= L) {
#pragma unroll
                    for (int h = 0; h < G; ++h) s[i][h] = -INFINITY;
                    vr[i] = make_uint4(0u, 0u, 0u, 0u);
                }
            }
        }

        float vf[LOADS][EPV];
#pragma unroll
        for (int i = 0; i < LOADS; ++i) chunk_to_f32<DT>(vr[i], vf[i]);

#pragma unroll
        for (int h = 0; h < G; ++h) {
            float mx = s[0][h];
#pragma unroll
            for (int i = 1; i < LOADS; ++i) mx = fmaxf(mx, s[i][h]);
            const float m_new = fmaxf(m[h], mx);
            const float ms = safe_max(m_new);
            const float corr = fast_exp2(m[h] - ms);
            float p[LOADS];
            float psum = 0.0f;
#pragma unroll
            for (int i = 0; i < LOADS; ++i) {
                p[i] = fast_exp2(s[i][h] - ms);
                psum += p[i];
            }
            l[h] = l[h] * corr + psum;
#pragma unroll
            for (int e = 0; e < EPV; ++e) {
                float x = acc[h][e] * corr;
#pragma unroll
                for (int i = 0; i < LOADS; ++i) x = fmaf(p[i], vf[i][e], x);
                acc[h][e] = x;
            }
            m[h] = m_new;
        }
    }

    // merge the TPL token rows of this wave (lanes c, c+LPT, c+2*LPT, ...)
#pragma unroll
    for (int off = LPT; off < kWave; off <<= 1) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float mo = __shfl_xor(m[h], off, kWave);
            const float lo = __shfl_xor(l[h], off, kWave);
            const float M = fmaxf(m[h], mo);
            const float Ms = safe_max(M);
            const float f = fast_exp2(m[h] - Ms);
            const float fo = fast_exp2(mo - Ms);
            l[h] = l[h] * f + lo * fo;
#pragma unroll
            for (int e = 0; e < EPV; ++e) {
                const float ao = __shfl_xor(acc[h][e], off, kWave);
                acc[h][e] = acc[h][e] * f + ao * fo;
            }
            m[h] = M;
        }
    }

    // merge the waves through LDS
    __shared__ float sm_m[kDecodeWaves][G];
    __shared__ float sm_l[kDecodeWaves][G];
    __shared__ float sm_acc[kDecodeWaves][G][D];
    if (r == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
#pragma unroll
            for (int e = 0; e < EPV; ++e) sm_acc[wave][h][c * EPV + e] = acc[h][e];
            if (c == 0) {
                sm_m[wave][h] = m[h];
                sm_l[wave][h] = l[h];
            }
        }
    }
    __syncthreads();

    const int hq0 = kv * G;
    for (int it = threadIdx.x; it < G * (D / 2); it += kDecodeWaves * kWave) {
        const int h = it / (D / 2);
        const int d = (it - h * (D / 2)) * 2;
        float M = sm_m[0][h];
#pragma unroll
        for (int w = 1; w < kDecodeWaves; ++w) M = fmaxf(M, sm_m[w][h]);
        const float Ms = safe_max(M);
        float den = 0.0f, n0 = 0.0f, n1 = 0.0f;
#pragma unroll
        for (int w = 0; w < kDecodeWaves; ++w) {
            const float f = fast_exp2(sm_m[w][h] - Ms);
            den = fmaf(sm_l[w][h], f, den);
            n0 = fmaf(sm_acc[w][h][d], f, n0);
            n1 = fmaf(sm_acc[w][h][d + 1], f, n1);
        }
        const size_t row = (size_t)seq * a.num_q_heads + hq0 + h;
        if (nparts == 1) {
            const float o0 = den > 0.0f ? n0 / den : 0.0f;
            const float o1 = den > 0.0f ? n1 / den : 0.0f;
            if constexpr (DT == 1) {
                reinterpret_cast<uint32_t*>(a.out)[(row * D + d) / 2] = pack_bf16x2(o0, o1);
            } else {
                reinterpret_cast<float2*>(a.out)[(row * D + d) / 2] = make_float2(o0, o1);
            }
        } else {
            const size_t slot = row * a.max_parts + part;
            reinterpret_cast<float2*>(a.ws_acc)[(slot * D + d) / 2] = make_float2(n0, n1);
            if (d == 0) reinterpret_cast<float2*>(a.ws_ml)[slot] = make_float2(M, den);
        }
    }
}

// Merge the partitions of one (sequence, query head): with M the largest
// partition max, out = sum_p acc_p 2^(m_p - M) / sum_p l_p 2^(m_p - M).
// Eight waves per (sequence, head), one pass: wave w takes partitions w,
// w + 8, ... kMergeU of them in flight per lane (lane: dims 2l, 2l + 1),
// keeping its own running max (what it summed so far is rescaled when a batch
// raises it); the eight partial states then meet in LDS.  A long context has
// hundreds of partitions (128K tokens in 512-token partitions: 256), so each
// wave takes them in one or two batches of loads rather than one at a time.
constexpr int kMergeWaves = 8;
constexpr int kMergeU = 16;

template <int DT, int D>
__global__ __launch_bounds__(kMergeWaves * kWave) void reduce_kernel(DecodeArgs a) {
    const int h = blockIdx.x;
    const int seq = blockIdx.y;
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = tid & (kWave - 1);
    int L = a.lens[seq];
    L = L < 0 ? 0 : (L > a.max_context ? a.max_context : L);
    const size_t row = (size_t)seq * a.num_q_heads + h;
    if (L == 0) {   // nothing to attend to: zeros (also written by the per-partition kernels)
        for (int d = tid * 2; d < D; d += kMergeWaves * kWave * 2) {
            if constexpr (DT == 1) reinterpret_cast<uint32_t*>(a.out)[(row * D + d) / 2] = 0u;
            else reinterpret_cast<float2*>(a.out)[(row * D + d) / 2] = make_float2(0.0f, 0.0f);
        }
        return;
    }
    const int nparts = (L + a.part_tokens - 1) / a.part_tokens;
    if (nparts <= 1) return;   // the decode kernel wrote this row itself

    const float2* ml = reinterpret_cast<const float2*>(a.ws_ml) + row * a.max_parts;
    const float2* acc = reinterpret_cast<const float2*>(a.ws_acc) + (row * a.max_parts) * (D / 2) + lane;
    const bool active = lane * 2 < D;
    float M = -INFINITY, den = 0.0f, n0 = 0.0f, n1 = 0.0f;
    for (int p0 = wave; p0 < nparts; p0 += kMergeWaves * kMergeU) {
        float2 mlu[kMergeU], xu[kMergeU];
#pragma unroll
        for (int u = 0; u < kMergeU; ++u) {
            const int p = p0 + u * kMergeWaves;
            const bool live = p < nparts;
            mlu[u] = live ? ml[p] : make_float2(-INFINITY, 0.0f);
            xu[u] = (live && active) ? acc[(size_t)p * (D / 2)] : make_float2(0.0f, 0.0f);
        }
        float mb = M;
#pragma unroll
        for (int u = 0; u < kMergeU; ++u) mb = fmaxf(mb, mlu[u].x);
        const float corr = fast_exp2(M - safe_max(mb));   // 0 for the first batch
        den *= corr;
        n0 *= corr;
        n1 *= corr;
        M = mb;
        const float Ms = safe_max(M);
#pragma unroll
        for (int u = 0; u < kMergeU; ++u) {
            const float f = fast_exp2(mlu[u].x - Ms);   // 0 for a missing partition
            den = fmaf(mlu[u].y, f, den);
            n0 = fmaf(xu[u].x, f, n0);
            n1 = fmaf(xu[u].y, f, n1);
        }
    }
    __shared__ float sm_m[kMergeWaves];
    __shared__ float sm_den[kMergeWaves];
    __shared__ float2 sm_n[kMergeWaves][kWave];
    if (lane == 0) {
        sm_m[wave] = M;
        sm_den[wave] = den;
    }
    sm_n[wave][lane] = make_float2(n0, n1);
    __syncthreads();
    if (wave != 0 || !active) return;
    float Mt = -INFINITY;
#pragma unroll
    for (int w = 0; w < kMergeWaves; ++w) Mt = fmaxf(Mt, sm_m[w]);
    const float Mts = safe_max(Mt);
    den = 0.0f;
    n0 = n1 = 0.0f;
#pragma unroll
    for (int w = 0; w < kMergeWaves; ++w) {
        const float f = fast_exp2(sm_m[w] - Mts);   // 0 for a wave that had no partition
        den = fmaf(sm_den[w], f, den);
        n0 = fmaf(sm_n[w][lane].x, f, n0);
        n1 = fmaf(sm_n[w][lane].y, f, n1);
    }
    const int d = lane * 2;
    const float o0 = den > 0.0f ? n0 / den : 0.0f;
    const float o1 = den > 0.0f ? n1 / den : 0.0f;
    if constexpr (DT == 1) {
        reinterpret_cast<uint32_t*>(a.out)[(row * D + d) / 2] = pack_bf16x2(o0, o1);
    } else {
        reinterpret_cast<float2*>(a.out)[(row * D + d) / 2] = make_float2(o0, o1);
    }
}

template <int DT, int D>
hipError_t launch_reduce(const DecodeArgs& a, hipStream_t stream) {
    if (a.max_parts <= 1) return hipSuccess;
    reduce_kernel<DT, D><<<dim3((unsigned)a.num_q_heads, (unsigned)a.num_seqs), dim3(kMergeWaves * kWave), 0, stream>>>(a);
    return hipGetLastError();
}

template <int DT, int D, int G>
hipError_t launch_tpl(const DecodeArgs& a, hipStream_t stream) {
    dim3 grid((unsigned)a.max_parts, (unsigned)a.num_kv_heads, (unsigned)a.num_seqs);
    decode_kernel<DT, D, G><<<grid, dim3(kDecodeWaves * kWave), 0, stream>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_reduce<DT, D>(a, stream);
}

template <int DT, int D>
hipError_t launch_group(const DecodeArgs& a, int group, hipStream_t stream) {
    switch (group) {
        case 1: return launch_tpl<DT, D, 1>(a, stream);
        case 2: return launch_tpl<DT, D, 2>(a, stream);
        case 4: return launch_tpl<DT, D, 4>(a, stream);
        case 8: return launch_tpl<DT, D, 8>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_partition_merge_bf16(const DecodeArgs& a, hipStream_t stream) {
    return launch_reduce<1, 128>(a, stream);
}

bool decode_shape_supported(int dtype, int head_dim, int group, int block_size) {
    if (!(dtype == 0 || dtype == 1 || dtype == 2) || !(head_dim == 64 || head_dim == 128) ||
        !(group == 1 || group == 2 || group == 4 || group == 8))
        return false;
    // the bf16 and FP8 / head_dim-128 kernels (matrix cores) walk 16-token
    // tiles of any block size 8..128; the vector-unit kernel is built for B = 16
    if (dtype == 2 && head_dim != 128) return false;
    if ((dtype == 1 || dtype == 2) && head_dim == 128)
        return block_size == 8 || block_size == 16 || block_size == 32 || block_size == 64 || block_size == 128;
    return block_size == kBlockTokens;
}

hipError_t launch_decode(const DecodeArgs& a, int dtype, int head_dim, hipStream_t stream) {
    if (a.num_seqs <= 0) return hipSuccess;
    const int group = a.num_q_heads / a.num_kv_heads;
    if (!decode_shape_supported(dtype, head_dim, group, a.block_size)) return hipErrorInvalidValue;
    if (dtype == 1 && head_dim == 128) {
        hipError_t e = launch_decode_bf16_mfma(a, group, stream);
        if (e != hipSuccess) return e;
        return launch_reduce<1, 128>(a, stream);
    }
    if (dtype == 2) {   // bf16 queries and outputs, so the bf16 merge
        hipError_t e = launch_decode_fp8_mfma(a, group, stream);
        if (e != hipSuccess) return e;
        return launch_reduce<1, 128>(a, stream);
    }
    if (dtype == 1) return launch_group<1, 64>(a, group, stream);
    return head_dim == 128 ? launch_group<0, 128>(a, group, stream) : launch_group<0, 64>(a, group, stream);
}

}  // namespace kvp
