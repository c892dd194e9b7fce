"""Pins of the oracle's swap (oracle.swap_out / oracle.swap_in) against what
fixes them independently of their own code:

* swapping blocks out and back into other blocks is the copy-on-write block
  copy (oracle.copy_blocks, pinned in test_oracle_pins.py): the same pools;
* out then back into the same blocks, after the pool was overwritten,
  restores it bit for bit (the round trip "aicassindra.com GPU paged KV cache",
  "Reclaiming memory: swap versus recompute" relies on);
* a record holds exactly the block's bytes of every layer: a pool of zeros
  with one block set to ones gives a record of ones and a buffer of zeros
  elsewhere; record sizes reproduce the pages' 2 MiB block and 1.25 GiB
  sequence (tests/golden/pages_numbers.json);
* FP8 scales travel with their block, as in the block copy.
"""
import json
import os

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = json.load(open(os.path.join(ROOT, "tests", "golden", "pages_numbers.json")))


def _pools(dtype, L=3, N=12, H=2, B=16, D=8, seed=0):
    rng = np.random.default_rng(seed)
    if dtype == np.uint16 or dtype == np.uint8:
        k = rng.integers(0, np.iinfo(dtype).max, (L, N, H, B, D), dtype=dtype)
        v = rng.integers(0, np.iinfo(dtype).max, (L, N, H, B, D), dtype=dtype)
    else:
        k = rng.standard_normal((L, N, H, B, D)).astype(dtype)
        v = rng.standard_normal((L, N, H, B, D)).astype(dtype)
    return k, v


@pytest.mark.parametrize("dtype", [np.float32, np.uint16])
def test_out_then_in_elsewhere_is_the_block_copy(dtype):
    k, v = _pools(dtype)
    src, dst = [3, 7, 0], [9, 1, 11]
    host = oracle.swap_out(k, v, src)
    k2, v2 = oracle.swap_in(k, v, dst, host)
    ek, ev = oracle.copy_blocks(k, v, list(zip(src, dst)))
    assert k2.tobytes() == ek.tobytes() and v2.tobytes() == ev.tobytes()


def test_round_trip_restores_overwritten_blocks():
    k, v = _pools(np.uint16, seed=1)
    blocks = [5, 2, 8, 10]
    host = oracle.swap_out(k, v, blocks)
    kc, vc = k.copy(), v.copy()
    kc[:, blocks] = 0xFFFF
    vc[:, blocks] = 0x7FC0
    k2, v2 = oracle.swap_in(kc, vc, blocks, host)
    assert k2.tobytes() == k.tobytes() and v2.tobytes() == v.tobytes()


def test_a_record_is_exactly_the_block_bytes():
    k = np.zeros((2, 6, 2, 16, 8), dtype=np.uint16)
    v = np.zeros_like(k)
    k[:, 4] = 1
    v[:, 4] = 1
    host = oracle.swap_out(k, v, [0, 4, 1]).reshape(3, -1)
    run = 2 * 16 * 8 * 2
    assert host.shape[1] == 2 * 2 * run
    assert not host[0].any() and not host[2].any()
    assert host[1].view(np.uint16).tolist() == [1] * (host.shape[1] // 2)
    # an index outside the pool leaves its record zero and is skipped on the way in
    host2 = oracle.swap_out(k, v, [4, 99, -1]).reshape(3, -1)
    assert host2[0].any() and not host2[1].any() and not host2[2].any()
    k3, v3 = oracle.swap_in(k, v, [99, -1, 2], np.ones(host2.size, dtype=np.uint8))
    assert k3[:, 2].view(np.uint8).min() == 1 and k3[:, :2].sum() == 0


def test_record_sizes_reproduce_the_pages():
    b = GOLDEN["kv_bytes_per_token_8b"]
    run = b["kv_heads"] * b["block_size"] * b["head_dim"] * b["elem_bytes"]
    assert oracle.swap_record_bytes(b["layers"], run) == b["expected_block_bytes"]
    g = GOLDEN["swap_4k_70b"]
    run = g["kv_heads"] * g["block_size"] * g["head_dim"] * g["elem_bytes"]
    total = oracle.swap_record_bytes(g["layers"], run) * (g["tokens"] // g["block_size"])
    assert total == g["expected_gib_each_way"] * 2**30
    # out and back: twice the sequence's KV bytes over the link
    assert GOLDEN["swap_cost_twice_kv"]["trips"] * total == 2 * g["tokens"] * 2 * g["layers"] * g["kv_heads"] * g["head_dim"] * g["elem_bytes"]


def test_fp8_scales_travel_with_their_block():
    k, v = _pools(np.uint8, L=2, N=10, H=3, D=128, seed=4)
    rng = np.random.default_rng(5)
    ks = rng.random((2, 10, 3)).astype(np.float32)
    vs = rng.random((2, 10, 3)).astype(np.float32)
    src, dst = [1, 6], [8, 2]
    host = oracle.swap_out(k, v, src, ks, vs)
    assert host.size == 2 * oracle.swap_record_bytes(2, 3 * 16 * 128, 3, fp8=True)
    k2, v2, ks2, vs2 = oracle.swap_in(k, v, dst, host, ks, vs)
    ek, ev = oracle.copy_blocks(k, v, list(zip(src, dst)))
    eks, evs = oracle.copy_blocks(ks[..., None, None], vs[..., None, None], list(zip(src, dst)))
    assert k2.tobytes() == ek.tobytes() and v2.tobytes() == ev.tobytes()
    assert ks2.tobytes() == eks[..., 0, 0].tobytes() and vs2.tobytes() == evs[..., 0, 0].tobytes()
