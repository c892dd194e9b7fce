"""Pins of the FP8 oracle (oracle/fp8.py) against things other than itself:
torch's float8_e4m3fn conversions (finite, in range), closed forms of the E4M3
format (ties, subnormals, saturation), the scale rule written out by hand, and
the fp64 C oracle on values that FP8 represents exactly."""
import math

import numpy as np
import pytest
import torch

import kvgen
import oracle
from oracle import fp8


def test_decode_matches_torch_and_the_format():
    codes = np.arange(256, dtype=np.uint8)
    d = fp8.e4m3_decode(codes)
    t = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    fin = np.isfinite(t)
    assert np.array_equal(d[fin], t[fin])
    assert list(np.nonzero(~np.isfinite(d))[0]) == [0x7F, 0xFF]
    assert d[0x7E] == 448.0 and d[0x01] == 2.0 ** -9 and d[0x08] == 2.0 ** -6 and d[0x38] == 1.0


def test_encode_matches_torch_in_range():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(50000) * 40, rng.uniform(-0.03, 0.03, 50000),
                        rng.uniform(-447, 447, 20000)]).astype(np.float32)
    x = x[np.abs(x) < 448]
    got = fp8.e4m3_encode(x)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, want)


def test_encode_ties_go_to_the_even_code_and_large_values_saturate():
    v = fp8.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = ((v[:-1] + v[1:]) / 2).astype(np.float32)          # exactly representable midpoints
    codes = fp8.e4m3_encode(mids)
    lower = np.arange(0x7E)
    assert np.array_equal(codes, np.where(lower % 2 == 0, lower, lower + 1))
    big = np.array([448, 449, 464, 480, 1e6, 3e38, -500, -448.0], dtype=np.float32)
    assert list(fp8.e4m3_encode(big)) == [0x7E] * 6 + [0xFE, 0xFE]
    assert fp8.e4m3_encode(np.float32(np.inf))[()] == 0x7E and fp8.e4m3_encode(np.float32(np.nan))[()] == 0x7F
    assert fp8.e4m3_encode(np.float32(-0.0))[()] == 0x80 and fp8.e4m3_encode(np.float32(2.0 ** -10))[()] == 0x00


def test_scale_rule_first_write_sets_it_later_writes_keep_it():
    N, H, B, D = 3, 2, 16, 8
    kc = np.zeros((N, H, B, D), np.uint8)
    vc = np.zeros_like(kc)
    ks = np.zeros((N, H), np.float32)
    vs = np.zeros_like(ks)
    rng = np.random.default_rng(1)
    rows = rng.standard_normal((4, H, D)).astype(np.float32)
    bits = kvgen.f32_to_bf16_bits(rows)
    f = fp8.bf16_bits_to_f32(bits)
    slots = np.array([16, 17, 18, 19])                         # rows 0..3 of block 1
    kc2, vc2, ks2, vs2 = fp8.scatter(kc, vc, ks, vs, bits, bits, slots, B)
    for h in range(H):
        amax = np.float32(np.abs(f[:, h, :]).max())
        assert ks2[1, h] == np.float32(amax / np.float32(448.0)) and vs2[1, h] == ks2[1, h]
    assert ks2[0].tolist() == [0, 0] and ks2[2].tolist() == [0, 0]
    # the largest element of each head lands exactly on the largest code
    for h in range(H):
        i = np.unravel_index(np.abs(f[:, h, :]).argmax(), f[:, h, :].shape)
        assert kc2[1, h, i[0], i[1]] & 0x7F == 0x7E
    # a later write (row 4) keeps the scale and saturates a value 10x the old amax
    big = (f[:1] * 0 + 10 * np.abs(f).max()).astype(np.float32)
    kc3, _, ks3, _ = fp8.scatter(kc2, vc2, ks2, vs2, kvgen.f32_to_bf16_bits(big), kvgen.f32_to_bf16_bits(big),
                                 np.array([20]), B)
    assert np.array_equal(ks3, ks2) and (kc3[1, :, 4, :] == 0x7E).all()


@pytest.mark.parametrize("B", [8, 128])
def test_scale_rule_covers_every_row_a_write_puts_into_a_block(B):
    """At any block size the write that fills row 0 sets the scale from all the
    rows it puts into that block (a prefill chunk filling it whole), and a row
    that opens the next block alone sets that block's scale from itself."""
    N, H, D = 4, 1, 8
    kc = np.zeros((N, H, B, D), np.uint8)
    ks = np.zeros((N, H), np.float32)
    rows = np.full((B + 1, H, D), 0.5, np.float32)
    rows[B - 1, 0, 3] = -96.0                  # the block's last row holds its largest magnitude
    rows[B, 0, :] = 2.0                        # row 0 of the next block, written by the same call
    bits = kvgen.f32_to_bf16_bits(rows)
    slots = np.concatenate([np.arange(2 * B, 3 * B), [B]])     # block 2 whole, then row 0 of block 1
    kc2, _, ks2, _ = fp8.scatter(kc, kc, ks, ks, bits, bits, slots, B)
    assert ks2[2, 0] == np.float32(96.0 / 448.0)
    assert ks2[1, 0] == np.float32(2.0 / 448.0)
    assert ks2[0, 0] == 0 and ks2[3, 0] == 0
    assert kc2[2, 0, B - 1, 3] == 0xFE                         # -96 is -448 x scale: the largest code
    assert (kc2[1, 0, 0, :] == 0x7E).all()                     # 2.0 alone: +448 x scale
    # 0.5 / (96 / 448) = 2.333..: the nearest E4M3 value is 2.25 (0x41)
    assert (kc2[2, 0, :B - 1, :] == 0x41).all()


def test_attention_matches_the_c_oracle_on_exact_values():
    """Codes times power-of-two scales are exact in bf16, so the FP8 path and the
    bf16 C oracle see the same numbers."""
    rng = np.random.default_rng(2)
    N, H, B, D, S, Hq = 10, 2, 16, 64, 3, 8
    codes = rng.integers(0, 0x70, size=(N, H, B, D)).astype(np.uint8) | (rng.integers(0, 2, (N, H, B, D)) << 7).astype(np.uint8)
    vcodes = rng.integers(0, 0x70, size=(N, H, B, D)).astype(np.uint8)
    ks = np.exp2(rng.integers(-8, -3, size=(N, H))).astype(np.float32)
    vs = np.exp2(rng.integers(-6, -1, size=(N, H))).astype(np.float32)
    kb = kvgen.f32_to_bf16_bits((fp8.e4m3_decode(codes) * ks[:, :, None, None]).astype(np.float32))
    vb = kvgen.f32_to_bf16_bits((fp8.e4m3_decode(vcodes) * vs[:, :, None, None]).astype(np.float32))
    assert np.array_equal(fp8.bf16_bits_to_f32(kb).astype(np.float64), fp8.e4m3_decode(codes) * ks[:, :, None, None])
    q = kvgen.f32_to_bf16_bits(rng.standard_normal((S, Hq, D)).astype(np.float32))
    tables = rng.permutation(N)[:9].reshape(3, 3).astype(np.int32)
    lens = np.array([40, 1, 33], np.int32)
    a = fp8.paged_attention(q, codes, vcodes, ks, vs, tables, lens, 0.125)
    b = oracle.paged_attention(q, kb, vb, "bf16", tables, lens, 0.125)
    assert np.abs(a - b).max() < 1e-12
