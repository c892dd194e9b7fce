"""CPU oracle for FP8 KV (E4M3 codes with one scale per (block, KV head)),
plain numpy, fp64 where the method is floating point.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle``: only the tests,
``__graft_entry__.smoke()`` and the benchmark's CPU-baseline leg use it.

The pages treat a 16-token block as a natural quantization group whose scales
travel with it ("PagedAttention, Internals First", "06 Open questions", the
paragraph on blocks as quantization groups; lattice-ai-eng "KV Cache &
PagedAttention", "5. Production tradeoffs", Quality: FP8 KV halves cache bytes
and decode traffic).  They fix no
format; this build reads them as:
  * codes: OCP E4M3 (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; no
    infinities; 0x7F / 0xFF are NaN; largest finite value 448);
  * one fp32 scale per (block, KV head) for K and one for V; a value is
    code * scale;
  * the write that covers row 0 of a block sets the block's scale to
    amax / 448 over the rows that write puts into that block (1.0 when they are
    all zero); later writes into the block keep it and saturate at +-448, so a
    block is never requantized;
  * quantizing is fp32 division by the scale, then round to nearest even among
    the E4M3 values, saturating at 448.

Parity status: decode and encode pinned against torch's float8_e4m3fn for
finite in-range values plus closed forms; the scatter's scale rule by closed
forms; attention against the fp64 C oracle on exactly representable values.
"""
from __future__ import annotations

import math

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """E4M3 code -> value (float64), from the bit fields."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = sign * (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = sign * (m / 8.0) * 2.0 ** -6
    out = np.where(e == 0, sub, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


_POS_CODES = np.arange(0x7F, dtype=np.uint8)          # 0x00..0x7E: the non-negative finite values
_POS_VALUES = e4m3_decode(_POS_CODES)                  # increasing


def e4m3_encode(x) -> np.ndarray:
    """float32 value -> E4M3 code: round to nearest, ties to the even code,
    saturate at +-448 (NaN -> 0x7F)."""
    with np.errstate(invalid="ignore"):   # signalling NaN inputs widen to NaN quietly
        v = np.asarray(x, dtype=np.float32).astype(np.float64)
    a = np.abs(v)
    i = np.clip(np.searchsorted(_POS_VALUES, a), 1, len(_POS_VALUES) - 1)   # a in [values[i-1], values[i]]
    lo, hi = _POS_VALUES[i - 1], _POS_VALUES[i]
    pick_hi = (a - lo > hi - a) | ((a - lo == hi - a) & ((_POS_CODES[i] & 1) == 0))
    code = np.where(pick_hi, _POS_CODES[i], _POS_CODES[i - 1]).astype(np.int64)
    code = np.where(a >= E4M3_MAX, 0x7E, code)
    code = np.where(a == 0.0, 0, code)
    code = code | np.where(np.signbit(v), 0x80, 0)
    code = np.where(np.isnan(v), 0x7F, code)
    return code.astype(np.uint8)


def bf16_bits_to_f32(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def block_scale(rows_f32: np.ndarray) -> np.float32:
    """Scale set by the first write into a block: amax / 448 over its rows (fp32), 1 if all zero."""
    amax = np.float32(np.max(np.abs(rows_f32))) if rows_f32.size else np.float32(0.0)
    return np.float32(amax / np.float32(E4M3_MAX)) if amax > 0 else np.float32(1.0)


def quantize_rows(rows_f32: np.ndarray, scale: np.float32) -> np.ndarray:
    return e4m3_encode((rows_f32.astype(np.float32) / np.float32(scale)).astype(np.float32))


def scatter(kc, vc, ks, vs, k_new_bits, v_new_bits, slots, block_size: int):
    """FP8 slot-mapping scatter.  kc / vc: uint8 [N][Hkv][B][D]; ks / vs: float32
    [N][Hkv]; k_new / v_new: bf16 bits [T][Hkv][D].  Returns new copies."""
    kc, vc, ks, vs = kc.copy(), vc.copy(), ks.copy(), vs.copy()
    N, H = ks.shape
    slots = np.asarray(slots, dtype=np.int64)
    kf = bf16_bits_to_f32(k_new_bits)
    vf = bf16_bits_to_f32(v_new_bits)
    valid = (slots >= 0) & (slots < N * block_size)
    blocks = np.where(valid, slots // block_size, -1)
    offs = np.where(valid, slots % block_size, -1)
    # scales: blocks whose row 0 is written now take amax / 448 over this write's rows in them
    for blk in np.unique(blocks[valid & (offs == 0)]):
        toks = np.nonzero(blocks == blk)[0]
        for h in range(H):
            ks[blk, h] = block_scale(kf[toks, h, :])
            vs[blk, h] = block_scale(vf[toks, h, :])
    for t in np.nonzero(valid)[0]:
        b, o = blocks[t], offs[t]
        for h in range(H):
            kc[b, h, o, :] = quantize_rows(kf[t, h, :], ks[b, h])
            vc[b, h, o, :] = quantize_rows(vf[t, h, :], vs[b, h])
    return kc, vc, ks, vs


def paged_attention(q_bits, kc, vc, ks, vs, block_tables, context_lens, scale: float) -> np.ndarray:
    """fp64 decode attention over dequantized K/V (code * scale) through the tables."""
    q = bf16_bits_to_f32(q_bits).astype(np.float64)
    S, Hq, D = q.shape
    N, Hkv, B, _ = kc.shape
    g = Hq // Hkv
    out = np.zeros((S, Hq, D), dtype=np.float64)
    kd = e4m3_decode(kc) * ks.astype(np.float64)[:, :, None, None]
    vd = e4m3_decode(vc) * vs.astype(np.float64)[:, :, None, None]
    for i in range(S):
        L = int(context_lens[i])
        if L <= 0:
            continue
        pos = np.arange(L)
        phys = np.asarray(block_tables[i])[pos // B]
        for kv in range(Hkv):
            K = kd[phys, kv, pos % B, :]
            V = vd[phys, kv, pos % B, :]
            for h in range(kv * g, (kv + 1) * g):
                s = K @ q[i, h] * scale
                w = np.exp(s - s.max())
                out[i, h] = (w @ V) / w.sum()
    return out
