"""Swap to pinned host memory and back on the GPU (kv_swap_out / kv_swap_in)
against oracle.swap_out / oracle.swap_in: the host buffer is bit-exact, the
round trip restores the pool bit for bit, swapping into other blocks equals
the oracle, FP8 scales travel with their blocks, and a sequence swapped out,
overwritten and swapped back into other blocks decodes to the same bits."""
import numpy as np
import pytest

import kvgen
import oracle
from parity_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu(gpu_available):
    yield


def _cuda(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _pinned(nbytes):
    import torch
    return torch.zeros(max(nbytes, 16), dtype=torch.uint8).pin_memory()


def _pool(dtype, layers, N, H, seed):
    import torch
    from paged_kv_cache_num_amd import KVPool
    rng = np.random.default_rng(seed)
    shape = (layers, N, H, 16, 128)
    if dtype == "fp8":
        pool = KVPool.allocate(num_layers=layers, num_blocks=N, block_size=16, num_kv_heads=H, head_dim=128,
                               dtype="fp8", device="cuda")
        k = rng.integers(0, 256, shape, dtype=np.uint8)
        v = rng.integers(0, 256, shape, dtype=np.uint8)
        ks = rng.random((layers, N, H)).astype(np.float32)
        vs = rng.random((layers, N, H)).astype(np.float32)
        pool.k.copy_(_cuda(k))
        pool.v.copy_(_cuda(v))
        pool.k_scale.copy_(_cuda(ks))
        pool.v_scale.copy_(_cuda(vs))
        return pool, (k, v, ks, vs)
    pool = KVPool.allocate(num_layers=layers, num_blocks=N, block_size=16, num_kv_heads=H, head_dim=128,
                           dtype=torch.bfloat16, device="cuda")
    k = rng.integers(0, 65536, shape, dtype=np.uint16)
    v = rng.integers(0, 65536, shape, dtype=np.uint16)
    pool.k.view(torch.int16).copy_(_cuda(k.view(np.int16)))
    pool.v.view(torch.int16).copy_(_cuda(v.view(np.int16)))
    return pool, (k, v)


def _host_state(pool, fp8):
    import torch
    if fp8:
        return (pool.k.cpu().numpy(), pool.v.cpu().numpy(), pool.k_scale.cpu().numpy(), pool.v_scale.cpu().numpy())
    return (pool.k.view(torch.int16).cpu().numpy().view(np.uint16), pool.v.view(torch.int16).cpu().numpy().view(np.uint16))


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_swap_out_in_matches_the_oracle(dtype):
    import torch
    say(f"swap {dtype}")
    fp8 = dtype == "fp8"
    layers, N, H = 3, 40, 8
    pool, state = _pool(dtype, layers, N, H, seed=7)
    out_blocks = np.array([17, 3, 29, 3, 39, 0, 55, -2], dtype=np.int32)   # a repeat and two outside the pool
    host = _pinned(pool.swap_bytes(out_blocks.size))
    assert host.numel() == pool.swap_bytes(out_blocks.size)
    host.fill_(0)
    pool.swap_out(_cuda(out_blocks), host)
    torch.cuda.synchronize()
    want = oracle.swap_out(*state[:2], out_blocks, *(state[2:] if fp8 else ()))
    got = host.numpy()
    assert got.tobytes() == want.tobytes(), f"{dtype}: host records differ"
    # overwrite the swapped blocks, swap back into the same blocks: the pool is restored
    back = np.array([17, 3, 29, 39, 0], dtype=np.int32)
    hb = _pinned(pool.swap_bytes(back.size))
    pool.swap_out(_cuda(back), hb)
    torch.cuda.synchronize()
    pool.k[:, back.tolist()] = 0x55 if fp8 else 0
    pool.v[:, back.tolist()] = 0x7F if fp8 else 0
    if fp8:
        pool.k_scale[:, back.tolist()] = 0.0
    pool.swap_in(_cuda(back), hb)
    torch.cuda.synchronize()
    for g, w in zip(_host_state(pool, fp8), state):
        assert g.tobytes() == w.tobytes(), f"{dtype}: round trip differs"
    # swap into other blocks
    dst = np.array([1, 2, 5, 6, 8], dtype=np.int32)
    pool.swap_in(_cuda(dst), hb)
    torch.cuda.synchronize()
    expect = oracle.swap_in(*state[:2], dst, hb.numpy(), *(state[2:] if fp8 else ()))
    for g, w in zip(_host_state(pool, fp8), expect):
        assert g.tobytes() == w.tobytes(), f"{dtype}: swap into other blocks differs"


def test_pageable_host_memory_is_refused():
    import torch
    from paged_kv_cache_num_amd import KVError
    pool, _ = _pool("bf16", 1, 8, 2, seed=1)
    host = torch.zeros(pool.swap_bytes(2), dtype=torch.uint8)   # not pinned
    with pytest.raises(KVError):
        pool.swap_out(_cuda(np.array([0, 1], dtype=np.int32)), host)
    with pytest.raises(KVError):
        pool.swap_in(_cuda(np.array([0, 1], dtype=np.int32)), host)


@pytest.mark.parametrize("fp8", [False, True])
def test_sequence_swapped_out_and_back_elsewhere_decodes_the_same(fp8):
    """Preempt one sequence (swap out), let another sequence's data overwrite
    its blocks, resume it into other free blocks (swap in, repoint the table):
    the decode of the batch is bitwise unchanged."""
    import torch
    from paged_kv_cache_num_amd import DecodeStep
    wl = kvgen.custom_workload(lengths=[700, 1500, 33, 260], num_q_heads=32, num_kv_heads=8, head_dim=128,
                               dtype="bf16", seed=61, variant="sharp", poison=False, num_blocks=260)
    state = kvgen.fp8_pool_state(wl, seed=3) if fp8 else None
    step = DecodeStep.from_workload(wl, fp8_pool=state, partition_size=0)
    step.attend()
    torch.cuda.synchronize()
    ref = step.out_host().copy()
    victim = 1
    nblk = -(-int(wl.context_lens[victim]) // wl.block_size)
    old = wl.block_tables[victim, :nblk].copy()
    used = set(np.unique(wl.block_tables[:, :]).tolist())
    free = np.array([b for b in range(wl.num_blocks) if b not in used][:nblk], dtype=np.int32)
    assert free.size == nblk
    host = _pinned(step.pool.swap_bytes(nblk))
    step.pool.swap_out(_cuda(old), host)
    torch.cuda.synchronize()
    step.pool.k[:, old.tolist()] = 0x7F if fp8 else 0   # another sequence reuses the freed blocks
    step.pool.v[:, old.tolist()] = 0x7F if fp8 else 0
    step.pool.swap_in(_cuda(free), host)
    tables = wl.block_tables.copy()
    tables[victim, :nblk] = free
    step.block_tables.copy_(_cuda(tables))
    step.attend()
    torch.cuda.synchronize()
    assert step.out_host().tobytes() == ref.tobytes()
