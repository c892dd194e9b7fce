"""A decode loop through the C ABI: many steps of one new token per sequence.

Each step takes a fresh block from the allocator fixture for every sequence
whose new token starts one (aicassindra.com "GPU paged KV cache", "The write
path: slot mapping and scatter": a block is taken when the previous one is
full; "PagedAttention, Internals First", "02 Block tables"), then appends the
token's K/V and attends in one call (paged_attention_decode_append).  The
oracle follows the same steps on the host: slot mapping, scatter, attention.
Every step's output is checked against the oracle's within the tolerance, and
after the last step the pool (FP8: codes and scales) must equal the oracle's
bit for bit, so that any row stored at a wrong place or with a wrong scale in
any step shows.  Table entries past a sequence's blocks name a block full of
NaN that no step may read.
"""
import math

import numpy as np
import pytest

import kvgen
import oracle
import oracle.fp8 as ofp8
from parity_util import TOL, say, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu(gpu_available):
    yield


START = [0, 1, 7, 15, 31, 63, 200]
STEPS = 40
HQ, HKV, D = 16, 4, 128

# (pool dtype, block size, partition size: 0 = balanced split)
CASES = [("bf16", 16, 0), ("bf16", 8, 0), ("bf16", 64, 0), ("bf16", 16, 64), ("fp8", 16, 0), ("fp8", 8, 0),
         ("fp8", 32, 0)]


def _bf16(rng, shape, scale):
    return kvgen.f32_to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))


@pytest.mark.parametrize("dtype,B,partition", CASES)
def test_decode_loop_matches_oracle_every_step(dtype, B, partition):
    import torch
    from paged_kv_cache_num_amd import KVPool

    fp8 = dtype == "fp8"
    say(f"decode loop {dtype} B={B} partition={partition}: {len(START)} sequences, {STEPS} steps")
    rng = np.random.default_rng(1000 + B + (7 if fp8 else 0) + partition)
    S = len(START)
    max_blocks = math.ceil((max(START) + STEPS) / B)
    N = S * max_blocks + 4
    poison = N - 1                                  # never handed out, never read
    alloc = kvgen.BlockAllocator(N - 1, order=rng.permutation(N - 1))
    rows = [[alloc.alloc() for _ in range(math.ceil(L / B))] for L in START]
    lens = np.array(START, dtype=np.int32)

    # pool contents before the loop: every existing token's rows (random values), poison block NaN
    if fp8:
        kc = kvgen.fp8_codes((N, HKV, B, D), np.random.SeedSequence(int(rng.integers(1 << 31))))
        vc = kvgen.fp8_codes((N, HKV, B, D), np.random.SeedSequence(int(rng.integers(1 << 31))))
        ks = ((0.5 + rng.random((N, HKV))) / 200).astype(np.float32)   # largest code about 1-3
        vs = ((0.5 + rng.random((N, HKV))) / 200).astype(np.float32)
        kc[poison] = 0x7F
        vc[poison] = 0x7F
    else:
        kp = _bf16(rng, (N, HKV, B, D), 1.0)
        vp = _bf16(rng, (N, HKV, B, D), 1.0)
        kp[poison] = 0x7FC0
        vp[poison] = 0x7FC0

    dev = torch.device("cuda")
    pool = KVPool.allocate(num_layers=1, num_blocks=N, block_size=B, num_kv_heads=HKV, head_dim=D,
                           dtype="fp8" if fp8 else torch.bfloat16)

    def upload():
        if fp8:
            pool.k.copy_(torch.from_numpy(kc.reshape(pool.k.shape)))
            pool.v.copy_(torch.from_numpy(vc.reshape(pool.v.shape)))
            pool.k_scale.copy_(torch.from_numpy(ks.reshape(pool.k_scale.shape)))
            pool.v_scale.copy_(torch.from_numpy(vs.reshape(pool.v_scale.shape)))
        else:
            pool.k.view(torch.int16).copy_(torch.from_numpy(kp.view(np.int16).reshape(pool.k.shape)))
            pool.v.view(torch.int16).copy_(torch.from_numpy(vp.view(np.int16).reshape(pool.v.shape)))

    upload()
    scale = 1.0 / math.sqrt(D)
    ws_cap = pool.workspace_bytes(S, HQ, max(START) + STEPS, partition)
    workspace = torch.empty(max(ws_cap, 1), dtype=torch.uint8, device=dev)
    out = torch.empty((S, HQ, D), dtype=torch.bfloat16, device=dev)
    worst = 0.0
    for step in range(STEPS):
        for i in range(S):                          # the new token's block, when it starts one
            if lens[i] % B == 0:
                rows[i].append(alloc.alloc())
        lens = lens + 1
        table = np.full((S, max_blocks), poison, dtype=np.int32)
        for i, r in enumerate(rows):
            table[i, :len(r)] = r
        q = _bf16(rng, (S, HQ, D), 1.0)
        k_new = _bf16(rng, (S, HKV, D), 1.0)
        v_new = _bf16(rng, (S, HKV, D), 1.0)
        max_len = int(lens.max())

        def t16(a):
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)

        pool.paged_attention_decode_append(0, out, t16(q), t16(k_new), t16(v_new),
                                           torch.from_numpy(table).to(dev), torch.from_numpy(lens).to(dev),
                                           scale=scale, max_context_len=max_len, partition_size=partition,
                                           workspace=workspace)
        torch.cuda.synchronize()

        slots = oracle.slot_mapping(table, B, N, np.arange(S, dtype=np.int32), lens - 1,
                                    np.ones(S, dtype=np.int32))
        if fp8:
            kc, vc, ks, vs = ofp8.scatter(kc, vc, ks, vs, k_new, v_new, slots, B)
            ref = ofp8.paged_attention(q, kc, vc, ks, vs, table, lens, scale)
        else:
            kp, vp = oracle.scatter(kp, vp, k_new, v_new, slots)
            ref = oracle.paged_attention(q, kp, vp, "bf16", table, lens, scale)
        got = to_f64(out.view(torch.int16).cpu().numpy().view(np.uint16), "bf16")
        assert np.isfinite(got).all(), f"step {step}: non-finite output (a NaN block was read)"
        err = float(np.abs(got - ref).max())
        worst = max(worst, err)
        assert err <= TOL["bf16"], f"step {step}: max |gpu - oracle| = {err:.3e}"

    say(f"  worst step: max |gpu - oracle| = {worst:.3e}; blocks in use {N - 1 - len(alloc.free)}")
    if fp8:
        assert pool.k.cpu().numpy().reshape(kc.shape).tobytes() == kc.tobytes(), "K codes differ"
        assert pool.v.cpu().numpy().reshape(vc.shape).tobytes() == vc.tobytes(), "V codes differ"
        assert pool.k_scale.cpu().numpy().reshape(ks.shape).tobytes() == ks.tobytes(), "K scales differ"
        assert pool.v_scale.cpu().numpy().reshape(vs.shape).tobytes() == vs.tobytes(), "V scales differ"
    else:
        gk = pool.k.view(torch.int16).cpu().numpy().view(np.uint16).reshape(kp.shape)
        gv = pool.v.view(torch.int16).cpu().numpy().view(np.uint16).reshape(vp.shape)
        assert gk.tobytes() == kp.tobytes(), "K pool differs"
        assert gv.tobytes() == vp.tobytes(), "V pool differs"
