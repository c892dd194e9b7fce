// Write path of FP8 pools: the slot-mapping scatter and the decode append
// with per-(block, KV head) scales.
//
// "PagedAttention, Internals First", "06 Open questions": a block is a natural
// quantization group, and a scale kept per block travels with it (copy-on-write
// copies included); sharing a block shares its scale, so a block must never be
// requantized once other rows depend on that scale.  The scale rule of these
// kernels: the write that puts row 0 of a block in place sets the block's K
// and V scales (one per KV head) to amax / 448 over the rows that write puts
// into the block (1.0 when they are all zero); every other write quantizes
// with the scale already stored, saturating at +-448.  Quantizing divides by
// the scale in fp32 and rounds to the nearest E4M3 code, ties to even.
//
// The scatter runs two kernels in stream order: fp8_scale_kernel finds the
// tokens that write row 0 of a block and sets those blocks' scales, then
// fp8_quantize_kernel writes every token's codes.  Slots are unique (the
// scatter's precondition), so a block has at most B writers, and when tokens
// t .. t+B-1 hold its slots B*blk .. B*blk+B-1 in order no other token can
// write it: that common case needs no search.
#include <math.h>

#include "device_common.hpp"
#include "fp8.hpp"
#include "fp8_rows.hpp"
#include "launch.hpp"

namespace kvp {

namespace {

constexpr int kD8 = 128;                 // head_dim of FP8 pools
constexpr int kRowWords = kD8 / 2;       // 32-bit words (bf16 pairs) per k_new / v_new row
constexpr int kRowChunks8 = kD8 / 16;    // 16-byte chunks per code row
constexpr int kQuantThreads = 256;

// One wave per (16-token chunk, KV head): grid (chunks, H), grid-stride over
// the chunks, so a wave usually has at most one block to open.  The wave finds
// the tokens of its chunk that write row 0 of a block and takes the amax of
// head h's K and V rows (lane l: dims 2l and 2l + 1) over every row this call
// writes into that block, sixteen rows at a time: lanes 0..15 list the writers
// of rows g .. g+15 (from the run that follows the token, else by searching
// the whole mapping, 512 slots per step: fp8_row_writers), and their 32 row
// loads go out together.
constexpr int kRowGroup = kFp8RowGroup;
constexpr int kScaleChunk = 16;

__global__ __launch_bounds__(kWave) void fp8_scale_kernel(ScatterArgs a) {
    const int lane = threadIdx.x;
    const int H = a.num_kv_heads;
    const int h = blockIdx.y;
    const int B = a.block_size;
    const int R = B < kRowGroup ? B : kRowGroup;   // rows per round
    const int64_t T = a.num_tokens;
    const uint32_t* kn = reinterpret_cast<const uint32_t*>(a.k_new);
    const uint32_t* vn = reinterpret_cast<const uint32_t*>(a.v_new);
    for (int64_t c0 = (int64_t)blockIdx.x * kScaleChunk; c0 < T; c0 += (int64_t)gridDim.x * kScaleChunk) {
        const int64_t t = c0 + lane;
        const int64_t slot = (lane < kScaleChunk && t < T) ? a.slot_mapping[t] : -1;
        uint64_t starts = __builtin_amdgcn_ballot_w64(slot >= 0 && slot < a.num_slots && slot % B == 0);
        while (starts) {
            const int j = __builtin_ctzll(starts);
            starts &= starts - 1;
            const int64_t first = fp8_readlane64(slot, j);   // slot of row 0
            const int64_t blk = first / B;
            float ak = 0.0f, av = 0.0f;
            for (int g = 0; g < B; g += R) {
                // lane i < R: the token writing row g + i of the block, or -1
                const int64_t tok = fp8_row_writers(a.slot_mapping, T, c0 + j + g, first + g, R, lane);
                uint32_t wk[kRowGroup], wv[kRowGroup];
#pragma unroll
                for (int i = 0; i < kRowGroup; ++i) {
                    const int64_t ti = fp8_readlane64(tok, i);
                    const size_t w = ((size_t)(ti < 0 ? 0 : ti) * H + h) * kRowWords + lane;
                    wk[i] = kn[w];
                    wv[i] = vn[w];
                }
#pragma unroll
                for (int i = 0; i < kRowGroup; ++i) {
                    if (fp8_readlane64(tok, i) >= 0) {
                        ak = abs_max2(wk[i], ak);
                        av = abs_max2(wv[i], av);
                    }
                }
            }
            ak = wave_max(ak);
            av = wave_max(av);
            if (lane == 0) {
                a.k_scale[blk * H + h] = e4m3_block_scale(ak);
                a.v_scale[blk * H + h] = e4m3_block_scale(av);
            }
        }
    }
}

// One thread per 16 codes: items ((token * 2 + {K,V}) * H + head) * 8 + chunk.
__global__ __launch_bounds__(kQuantThreads) void fp8_quantize_kernel(ScatterArgs a) {
    // workgroup y: one token at a time (its slot read once); x: its K and V
    // code chunks ({K,V} * H + head) * kRowChunks8 + chunk, in 32 bits
    const int H = a.num_kv_heads;
    const int per_head = H * kRowChunks8;
    for (int64_t t = blockIdx.y; t < a.num_tokens; t += gridDim.y) {
        const int64_t slot = a.slot_mapping[t];
        if (slot < 0 || slot >= a.num_slots) continue;
        const int64_t blk = slot / a.block_size;
        const int off = (int)(slot - blk * a.block_size);
        for (int item = blockIdx.x * kQuantThreads + threadIdx.x; item < 2 * per_head;
             item += gridDim.x * kQuantThreads) {
            const int which = item >= per_head;
            const int rem = item - which * per_head;
            const int h = rem / kRowChunks8;
            const int c = rem - h * kRowChunks8;
            const float s = (which == 0 ? a.k_scale : a.v_scale)[blk * H + h];
            const uint4* src = reinterpret_cast<const uint4*>(which == 0 ? a.k_new : a.v_new) +
                               ((t * H + h) * (kD8 / 8) + 2 * c);
            const uint4 x0 = src[0], x1 = src[1];
            uint4 o;
            o.x = bf16x2_to_e4m3x2(x0.x, s) | (bf16x2_to_e4m3x2(x0.y, s) << 16);
            o.y = bf16x2_to_e4m3x2(x0.z, s) | (bf16x2_to_e4m3x2(x0.w, s) << 16);
            o.z = bf16x2_to_e4m3x2(x1.x, s) | (bf16x2_to_e4m3x2(x1.y, s) << 16);
            o.w = bf16x2_to_e4m3x2(x1.z, s) | (bf16x2_to_e4m3x2(x1.w, s) << 16);
            uint4* dst = reinterpret_cast<uint4*>(which == 0 ? a.k_layer : a.v_layer);
            dst[((blk * H + h) * a.block_size + off) * kRowChunks8 + c] = o;
        }
    }
}

// Decode append: one wave per (sequence, {K,V}, KV head), four per workgroup;
// lane l quantizes dims 2l and 2l + 1.  The row goes to position L - 1; if that
// is row 0 of its block, this row alone sets the block's scale.
constexpr int kAppendWaves = 4;

__global__ __launch_bounds__(kAppendWaves * kWave) void fp8_append_kernel(AppendArgs a) {
    const int lane = threadIdx.x & (kWave - 1);
    const int H = a.num_kv_heads;
    const int64_t item = (int64_t)blockIdx.x * kAppendWaves + threadIdx.x / kWave;   // (seq * 2 + which) * H + h
    if (item >= (int64_t)a.num_seqs * 2 * H) return;
    const int64_t seq = item / (2 * H);
    const int which = (int)((item / H) & 1);
    const int h = (int)(item - (seq * 2 + which) * H);
    int L = a.lens[seq];
    L = L < 0 ? 0 : (L > a.max_context ? a.max_context : L);
    if (L == 0) return;
    const int pos = L - 1;
    const int64_t block = a.tables[seq * a.max_blocks + pos / a.block_size];
    if (block < 0 || block >= a.num_blocks) return;
    const int j = pos % a.block_size;
    const uint32_t* src = reinterpret_cast<const uint32_t*>(which == 0 ? a.k_new : a.v_new) + (seq * H + h) * kRowWords;
    uint16_t* dst = reinterpret_cast<uint16_t*>(which == 0 ? a.k_layer : a.v_layer) +
                    ((block * H + h) * a.block_size + j) * (kD8 / 2);
    fp8_store_row(src, dst, (which == 0 ? a.k_scale : a.v_scale) + block * H + h, j == 0, lane);
}

}  // namespace

hipError_t launch_scatter_fp8(const ScatterArgs& a, hipStream_t stream) {
    if (a.num_tokens <= 0) return hipSuccess;
    if ((a.block_size != 8 && a.block_size != 16 && a.block_size != 32 && a.block_size != 64 &&
         a.block_size != 128) || a.num_kv_heads <= 0 || a.num_kv_heads > 65535)
        return hipErrorInvalidValue;
    int64_t chunks = (a.num_tokens + kScaleChunk - 1) / kScaleChunk;
    if (chunks > 8192) chunks = 8192;   // grid-stride over the rest
    fp8_scale_kernel<<<dim3((unsigned)chunks, (unsigned)a.num_kv_heads), dim3(kWave), 0, stream>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned gx = (unsigned)((2 * a.num_kv_heads * kRowChunks8 + kQuantThreads - 1) / kQuantThreads);
    const unsigned gy = (unsigned)(a.num_tokens < 65535 ? a.num_tokens : 65535);   // grid-stride over the rest
    fp8_quantize_kernel<<<dim3(gx, gy), dim3(kQuantThreads), 0, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_append_fp8(const AppendArgs& a, hipStream_t stream) {
    if (a.num_seqs <= 0) return hipSuccess;
    const int64_t items = (int64_t)a.num_seqs * 2 * a.num_kv_heads;
    const int64_t blocks = (items + kAppendWaves - 1) / kAppendWaves;
    fp8_append_kernel<<<dim3((unsigned)blocks), dim3(kAppendWaves * kWave), 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace kvp
