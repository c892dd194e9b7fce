// Measurement probe: a plain 16-byte-vector device copy of known size, used to
// calibrate HBM byte counters and as the achievable-bandwidth reference.
#include <hip/hip_runtime.h>

#include "fp8.hpp"
#include "kvpool_probe.h"
#include "launch.hpp"
#include "split.hpp"

namespace {

constexpr int kCopyThreads = 256;

__global__ __launch_bounds__(kCopyThreads) void copy_kernel(uint4* __restrict__ dst, const uint4* __restrict__ src,
                                                            uint64_t n) {
    const uint64_t stride = (uint64_t)gridDim.x * kCopyThreads;
    for (uint64_t i = (uint64_t)blockIdx.x * kCopyThreads + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

constexpr int kReadBlocks = 256 * 32;   // 32 workgroups per compute unit, grid-stride

__global__ __launch_bounds__(kCopyThreads) void read_kernel(const uint4* __restrict__ src, uint64_t n,
                                                            uint32_t* __restrict__ sink) {
    const uint64_t stride = (uint64_t)gridDim.x * kCopyThreads;
    uint32_t acc = 0;
    for (uint64_t i = (uint64_t)blockIdx.x * kCopyThreads + threadIdx.x; i < n; i += stride) {
        const uint4 x = src[i];   // a plain (allocating) load: reading evicts what the caches held
        acc ^= x.x ^ x.y ^ x.z ^ x.w;
    }
    // fold the wave, then one word per workgroup
    for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
    __shared__ uint32_t part[kCopyThreads / 64];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t v = 0;
        for (int w = 0; w < kCopyThreads / 64; ++w) v ^= part[w];
        sink[blockIdx.x % (65536 / 4)] = v;
    }
}

// Table walk of the balanced decode split without the K/V stream: every worker
// scans the lengths, takes the same slice as the decode kernel and reads its
// block-table entries the same way (one vector load per 64 entries of a
// (sequence, KV head) piece).  Grouped: slice s runs on XCD s / (W / 8), so
// the KV heads of a sequence, which are neighbours in the tile list, share
// one XCD's L2 instead of being spread over all eight.
template <bool kGrouped>
__global__ __launch_bounds__(64) void table_walk_kernel(const int32_t* __restrict__ tables, int32_t max_blocks,
                                                        const int32_t* __restrict__ lens, int32_t S, int32_t Hkv,
                                                        int32_t max_context, uint32_t* __restrict__ sink) {
    const int lane = threadIdx.x;
    const int64_t W = gridDim.x;
    const int64_t w = blockIdx.x;
    const int64_t s = kGrouped ? (w % 8) * (W / 8) + w / 8 : w;
    auto clamp = [&](int L) { return L < 0 ? 0 : (L > max_context ? max_context : L); };
    auto tiles = [&](int i) -> int64_t {   // split positions of sequence i
        return i < S ? (int64_t)Hkv * kvp::walk_span((clamp(lens[i]) + kvp::kBlockTokens - 1) / kvp::kBlockTokens, kvp::kBf16PieceCost) : 0;
    };
    int64_t T = 0;
    for (int b = 0; b < S; b += 64) {
        int64_t x = tiles(b + lane);
        for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
        T += x;
    }
    const kvp::SplitConsts sc = kvp::split_consts(W, kvp::kBf16SliceWeights);
    int64_t t = kvp::slice_start(s, T, sc);
    const int64_t t_end = kvp::slice_start(s + 1, T, sc);
    uint32_t acc = 0;
    // the sequence holding tile t, 64 sequences per step
    int seq = S;
    int64_t first = 0;   // first tile of sequence seq
    int64_t carry = 0;
    for (int b = 0; b < S && seq == S && t < t_end; b += 64) {
        const int64_t nt = tiles(b + lane);
        int64_t incl = nt;
        for (int off = 1; off < 64; off <<= 1) {
            const int64_t y = __shfl_up(incl, off, 64);
            if (lane >= off) incl += y;
        }
        const int64_t ex = carry + incl - nt;
        const uint64_t bal = __builtin_amdgcn_ballot_w64(nt > 0 && ex <= t && t < ex + nt);
        if (bal) {
            const int j = __builtin_ctzll(bal);
            seq = b + j;
            first = __shfl(ex, j, 64);
        }
        carry += __shfl(incl, 63, 64);
    }
    seq = __builtin_amdgcn_readfirstlane(seq);
    for (; seq < S && t < t_end; ++seq) {
        const int L = __builtin_amdgcn_readfirstlane(clamp(lens[seq]));
        const int nblk = (L + kvp::kBlockTokens - 1) / kvp::kBlockTokens;
        const int64_t span = kvp::walk_span(nblk, kvp::kBf16PieceCost);
        const int64_t seg_end = first + (int64_t)Hkv * span;
        while (t < t_end && t < seg_end) {
            // walk kv of this sequence: its tile b sits at position kBf16PieceCost + b of its span
            const int64_t off = t - first;
            const int kv = (int)(off / span);
            const int b = kvp::first_tile_at(off - (int64_t)kv * span, kvp::kBf16PieceCost);
            const int64_t tb = first + (int64_t)kv * span + kvp::kBf16PieceCost + b;
            const int n = (int)max((int64_t)0, min((int64_t)(nblk - b), t_end - tb));
            const int32_t* trow = tables + (size_t)seq * max_blocks + b;
            for (int k0 = 0; k0 < n; k0 += 64)
                if (k0 + lane < n) acc ^= (uint32_t)trow[k0 + lane] + (uint32_t)kv;
            t = first + (int64_t)(kv + 1) * span;
        }
        first = seg_end;
    }
    for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
    if (lane == 0) sink[w] = acc;
}

// E4M3 conversions as the FP8 pool kernels do them.  Widening: thread i takes
// codes 2i and 2i + 1 as one 16-bit word, in the low half of the operand for
// even i and the high half for odd i, so both word selects are exercised.
__global__ __launch_bounds__(256) void e4m3_widen_kernel(const uint8_t* __restrict__ codes, uint16_t* __restrict__ out,
                                                         int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (2 * i >= n) return;
    const bool second = 2 * i + 1 < n;
    const uint32_t w = (uint32_t)codes[2 * i] | (second ? (uint32_t)codes[2 * i + 1] << 8 : 0u);
    const uint32_t r = (i & 1) ? kvp::e4m3x2_to_bf16x2<true>(w << 16) : kvp::e4m3x2_to_bf16x2<false>(w);
    out[2 * i] = (uint16_t)r;
    if (second) out[2 * i + 1] = (uint16_t)(r >> 16);
}

__global__ __launch_bounds__(256) void e4m3_encode_kernel(const float* __restrict__ x, uint8_t* __restrict__ out,
                                                          int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) out[i] = (uint8_t)kvp::f32_to_e4m3(x[i]);
}

}  // namespace

extern "C" kv_status kv_probe_e4m3_to_bf16(const void* codes, void* out_bf16, int64_t n, void* stream) {
    if (n < 0 || (n > 0 && (!codes || !out_bf16)) || (reinterpret_cast<uintptr_t>(out_bf16) & 1u))
        return KV_ERR_INVALID_ARGUMENT;
    if (n == 0) return KV_OK;
    const int64_t threads = (n + 1) / 2;
    if ((threads + 255) / 256 > 0x7FFFFFFF) return KV_ERR_INVALID_ARGUMENT;
    e4m3_widen_kernel<<<dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<const uint8_t*>(codes), static_cast<uint16_t*>(out_bf16), n);
    return hipGetLastError() == hipSuccess ? KV_OK : KV_ERR_HIP;
}

extern "C" kv_status kv_probe_f32_to_e4m3(const float* x, void* out_codes, int64_t n, void* stream) {
    if (n < 0 || (n > 0 && (!x || !out_codes)) || (reinterpret_cast<uintptr_t>(x) & 3u)) return KV_ERR_INVALID_ARGUMENT;
    if (n == 0) return KV_OK;
    if ((n + 255) / 256 > 0x7FFFFFFF) return KV_ERR_INVALID_ARGUMENT;
    e4m3_encode_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, static_cast<hipStream_t>(stream)>>>(
        x, static_cast<uint8_t*>(out_codes), n);
    return hipGetLastError() == hipSuccess ? KV_OK : KV_ERR_HIP;
}

extern "C" kv_status kv_probe_table_walk(const int32_t* block_tables, int32_t max_blocks_per_seq,
                                         const int32_t* context_lens, int32_t num_seqs, int32_t num_kv_heads,
                                         int32_t max_context_len, int32_t xcd_grouped, void* sink,
                                         uint64_t sink_bytes, void* stream) {
    if (!block_tables || !context_lens || !sink || num_seqs < 0 || num_kv_heads <= 0 || max_context_len < 0 ||
        max_blocks_per_seq <= 0 || (int64_t)max_context_len > (int64_t)max_blocks_per_seq * kvp::kBlockTokens ||
        (reinterpret_cast<uintptr_t>(sink) & 3u))
        return KV_ERR_INVALID_ARGUMENT;
    const int workers = kvp::streamk_workers(4, false);
    if (workers <= 0 || workers % 8 != 0 || sink_bytes < (uint64_t)workers * 4u) return KV_ERR_INVALID_ARGUMENT;
    if (num_seqs == 0) return KV_OK;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (xcd_grouped)
        table_walk_kernel<true><<<dim3((unsigned)workers), dim3(64), 0, st>>>(
            block_tables, max_blocks_per_seq, context_lens, num_seqs, num_kv_heads, max_context_len,
            static_cast<uint32_t*>(sink));
    else
        table_walk_kernel<false><<<dim3((unsigned)workers), dim3(64), 0, st>>>(
            block_tables, max_blocks_per_seq, context_lens, num_seqs, num_kv_heads, max_context_len,
            static_cast<uint32_t*>(sink));
    return hipGetLastError() == hipSuccess ? KV_OK : KV_ERR_HIP;
}

extern "C" kv_status kv_probe_read(const void* src, uint64_t bytes, void* sink, void* stream) {
    if (!src || !sink || (bytes & 15u) || (reinterpret_cast<uintptr_t>(src) & 15u) || (reinterpret_cast<uintptr_t>(sink) & 3u))
        return KV_ERR_INVALID_ARGUMENT;
    const uint64_t n = bytes / 16;
    if (n == 0) return KV_OK;
    uint64_t blocks = (n + kCopyThreads - 1) / kCopyThreads;
    if (blocks > kReadBlocks) blocks = kReadBlocks;
    read_kernel<<<dim3((unsigned)blocks), dim3(kCopyThreads), 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<const uint4*>(src), n, static_cast<uint32_t*>(sink));
    return hipGetLastError() == hipSuccess ? KV_OK : KV_ERR_HIP;
}

extern "C" kv_status kv_probe_copy(void* dst, const void* src, uint64_t bytes, void* stream) {
    if (!dst || !src || (bytes & 15u) || ((reinterpret_cast<uintptr_t>(dst) | reinterpret_cast<uintptr_t>(src)) & 15u))
        return KV_ERR_INVALID_ARGUMENT;
    const uint64_t n = bytes / 16;
    if (n == 0) return KV_OK;
    uint64_t blocks = (n + kCopyThreads - 1) / kCopyThreads;
    if (blocks > 256 * 64) blocks = 256 * 64;   // 64 workgroups per CU, grid-stride for the rest
    copy_kernel<<<dim3((unsigned)blocks), dim3(kCopyThreads), 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<uint4*>(dst), static_cast<const uint4*>(src), n);
    return hipGetLastError() == hipSuccess ? KV_OK : KV_ERR_HIP;
}
