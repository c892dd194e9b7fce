"""Copy-on-write on the GPU: kv_copy_blocks is a bit copy of whole blocks in every
layer, and a fork -> divergent append -> attend step through it matches the
oracle (copy, scatter, fp64 attention) with every table seeing its own data."""
import math

import numpy as np
import pytest

import kvgen
import oracle
from parity_util import TOL, max_err, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu(gpu_available):
    yield


def _pool(dtype, layers, N, H, D, seed):
    import torch
    from paged_kv_cache_num_amd import KVPool
    from paged_kv_cache_num_amd.step import to_device
    rng = np.random.default_rng(seed)
    shape = (layers, N, H, 16, D)
    kh = rng.standard_normal(shape).astype(np.float32)
    vh = rng.standard_normal(shape).astype(np.float32)
    if dtype == "bf16":
        kh, vh = kvgen.f32_to_bf16_bits(kh), kvgen.f32_to_bf16_bits(vh)
    pool = KVPool.allocate(num_layers=layers, num_blocks=N, block_size=16, num_kv_heads=H, head_dim=D,
                           dtype=torch.float32 if dtype == "f32" else torch.bfloat16, device="cuda")
    for li in range(layers):
        pool.k[li].copy_(to_device(kh[li], dtype))
        pool.v[li].copy_(to_device(vh[li], dtype))
    return pool, kh, vh


@pytest.mark.parametrize("dtype,layers,H,D", [("bf16", 3, 8, 128), ("f32", 2, 2, 64)])
def test_copy_blocks_is_a_bit_copy_of_every_layer(dtype, layers, H, D):
    import torch
    from paged_kv_cache_num_amd.step import to_host
    say(f"copy_blocks dtype={dtype} layers={layers} H={H} D={D}")
    N = 40
    pool, kh, vh = _pool(dtype, layers, N, H, D, seed=5)
    rng = np.random.default_rng(6)
    perm = rng.permutation(N)
    pairs = [(int(perm[i]), int(perm[20 + i])) for i in range(12)]     # distinct sources and destinations
    pairs += [(-1, 3), (5, N), (N + 7, 2)]                             # outside the pool: skipped
    dp = torch.tensor(pairs, dtype=torch.int32, device="cuda")
    pool.copy_blocks(dp)
    pool.copy_blocks(dp[:0])                                            # no pairs: nothing queued
    torch.cuda.synchronize()
    ek, ev = oracle.copy_blocks(kh, vh, pairs)
    for li in range(layers):
        assert to_host(pool.k[li], dtype).tobytes() == ek[li].tobytes(), f"K layer {li}"
        assert to_host(pool.v[li], dtype).tobytes() == ev[li].tobytes(), f"V layer {li}"


def test_fork_diverge_attend_matches_the_oracle():
    """Four sequences share a 100-token prompt (6 full blocks and a 4-token tail
    block); each appends one token at position 100.  The block manager copies
    the shared tail for the first three writers; the device copies, the
    scatter writes each token into its own block, and attention over the four
    tables matches the oracle.  The prompt's full blocks stay shared."""
    import torch
    from paged_kv_cache_num_amd import KVPool, kv_build_slot_mapping
    from paged_kv_cache_num_amd.step import to_device, to_host
    say("fork -> copy-on-write append -> decode")
    dtype, H, Hq, D, N, B = "bf16", 8, 32, 128, 48, 16
    pool, kh, vh = _pool(dtype, 1, N, H, D, seed=7)
    kh, vh = kh[0], vh[0]
    alloc = kvgen.BlockAllocator(N, order=np.random.default_rng(8).permutation(N))
    parent = [alloc.alloc() for _ in range(7)]
    rows = [alloc.fork(parent) for _ in range(3)] + [parent]
    pairs = [p for p in (alloc.cow_for_append(r, 100, B) for r in rows) if p is not None]
    assert len(pairs) == 3 and alloc.refcount[parent[0]] == 4
    S = len(rows)
    MB = 8
    tables = np.zeros((S, MB), dtype=np.int32)
    for i, r in enumerate(rows):
        tables[i, :len(r)] = r
    lens = np.full(S, 101, dtype=np.int32)
    rng = np.random.default_rng(9)
    q = kvgen.f32_to_bf16_bits(rng.standard_normal((S, Hq, D)).astype(np.float32))
    k_new = kvgen.f32_to_bf16_bits(rng.standard_normal((S, H, D)).astype(np.float32))
    v_new = kvgen.f32_to_bf16_bits(rng.standard_normal((S, H, D)).astype(np.float32))
    slots = kv_build_slot_mapping(tables, B, N, np.arange(S, dtype=np.int32), lens - 1, np.ones(S, dtype=np.int32))
    # GPU: copy, scatter, attend
    pool.copy_blocks(torch.tensor(pairs, dtype=torch.int32, device="cuda"))
    pool.reshape_and_cache(0, to_device(k_new, dtype), to_device(v_new, dtype), to_device(slots, "i64"))
    out = torch.empty((S, Hq, D), dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(max(16, pool.workspace_bytes(S, Hq, 101, 0)), dtype=torch.uint8, device="cuda")
    scale = 1.0 / math.sqrt(D)
    pool.paged_attention_decode(0, out, to_device(q, dtype), to_device(tables, "i32"), to_device(lens, "i32"),
                                scale=scale, max_context_len=101, partition_size=0, workspace=ws)
    torch.cuda.synchronize()
    # oracle: the same three steps
    ek, ev = oracle.copy_blocks(kh, vh, pairs)
    ek, ev = oracle.scatter(ek, ev, k_new, v_new, slots)
    ref = oracle.paged_attention(q, ek, ev, dtype, tables, lens, scale)
    assert to_host(pool.k[0], dtype).tobytes() == ek.tobytes()
    assert to_host(pool.v[0], dtype).tobytes() == ev.tobytes()
    err = max_err(to_host(out, dtype), ref, dtype)
    say(f"  max |gpu - oracle| = {err:.3e}")
    assert err <= TOL[dtype]
    # the four sequences share 100 tokens and differ only in the last one
    assert len({int(t[6]) for t in tables}) == 4 and len({tuple(t[:6]) for t in tables}) == 1
