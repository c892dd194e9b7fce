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


# Continuous batching: requests join the decode batch after their prompt was
# stored in chunks by the step call beside the other sequences' decode
# (paged_attention_decode_step), and finished requests give their blocks back,
# which later prompts reuse with their stale rows still in place.
#   request: (prompt tokens, first prefill step, chunk size, step after which it finishes or None)
REQUESTS = [(3, None, 0, None), (40, None, 0, 9), (17, None, 0, None), (100, None, 0, 15), (64, None, 0, None),
            (300, 4, 128, None), (150, 10, 100, None)]
CB_STEPS = 24
CB_CASES = [("bf16", 16, 0), ("bf16", 8, 0), ("bf16", 16, 128), ("fp8", 16, 0), ("fp8", 64, 0)]


@pytest.mark.parametrize("dtype,B,partition", CB_CASES)
def test_continuous_batching_with_prefill_chunks_and_block_reuse(dtype, B, partition):
    import torch
    from paged_kv_cache_num_amd import KVPool, kv_build_slot_mapping

    fp8 = dtype == "fp8"
    say(f"continuous batching {dtype} B={B} partition={partition}: {len(REQUESTS)} requests, {CB_STEPS} steps")
    rng = np.random.default_rng(2000 + B + (7 if fp8 else 0) + partition)
    N = math.ceil(1200 / B) + 16
    poison = N - 1
    alloc = kvgen.BlockAllocator(N - 1, order=rng.permutation(N - 1))
    max_blocks = math.ceil((max(p for p, *_ in REQUESTS) + CB_STEPS) / B)
    rows = {}      # request -> its blocks
    lens = {}      # request -> tokens stored
    batch = []     # requests decoding, in batch order
    for r, (P, first, _, _) in enumerate(REQUESTS):
        if first is None:   # already prefilled before the loop (its rows written below)
            rows[r] = [alloc.alloc() for _ in range(math.ceil(P / B))]
            lens[r] = P
            batch.append(r)

    if fp8:
        kc = kvgen.fp8_codes((N, HKV, B, D), np.random.SeedSequence(int(rng.integers(1 << 31))))
        vc = kvgen.fp8_codes((N, HKV, B, D), np.random.SeedSequence(int(rng.integers(1 << 31))))
        ks = ((0.5 + rng.random((N, HKV))) / 200).astype(np.float32)
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
    if fp8:
        for t, a in ((pool.k, kc), (pool.v, vc), (pool.k_scale, ks), (pool.v_scale, vs)):
            t.copy_(torch.from_numpy(a.reshape(t.shape)))
    else:
        pool.k.view(torch.int16).copy_(torch.from_numpy(kp.view(np.int16).reshape(pool.k.shape)))
        pool.v.view(torch.int16).copy_(torch.from_numpy(vp.view(np.int16).reshape(pool.v.shape)))

    def t16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    scale = 1.0 / math.sqrt(D)
    ws_cap = max(pool.workspace_bytes(S_, HQ, max_blocks * B, partition) for S_ in range(1, len(REQUESTS) + 1))
    workspace = torch.empty(max(ws_cap, 1), dtype=torch.uint8, device=dev)
    worst, chunks, reused = 0.0, 0, 0
    freed = set()
    for step in range(CB_STEPS):
        # the prompt chunk stored this step, if a request is being prefilled
        pre = None
        for r, (P, first, chunk, _) in enumerate(REQUESTS):
            if first is not None and r not in batch and first <= step and lens.get(r, 0) < P:
                pre = r
        if pre is not None:
            P, _, chunk, _ = REQUESTS[pre]
            c0 = lens.get(pre, 0)
            n = min(chunk, P - c0)
            rows.setdefault(pre, [])
            while len(rows[pre]) * B < c0 + n:
                b = alloc.alloc()
                reused += b in freed
                rows[pre].append(b)
        for r in batch:     # each decoding request's new token, in a fresh block when it starts one
            if lens[r] % B == 0:
                rows[r].append(alloc.alloc())
            lens[r] += 1
        S = len(batch)
        table = np.full((S + 1, max_blocks), poison, dtype=np.int32)   # the batch, then the prefilling request
        for i, r in enumerate(batch):
            table[i, :len(rows[r])] = rows[r]
        L = np.array([lens[r] for r in batch], dtype=np.int32)
        q = _bf16(rng, (S, HQ, D), 1.0)
        k_new = _bf16(rng, (S, HKV, D), 1.0)
        v_new = _bf16(rng, (S, HKV, D), 1.0)
        ws_seq = list(range(S))
        ws_start = list(L - 1)
        ws_count = [1] * S
        k_rows = v_rows = np.zeros((0, HKV, D), dtype=np.uint16)
        if pre is not None:
            table[S, :len(rows[pre])] = rows[pre]
            k_rows = _bf16(rng, (n, HKV, D), 1.0)
            v_rows = _bf16(rng, (n, HKV, D), 1.0)
            ws_seq.append(S)
            ws_start.append(c0)
            ws_count.append(n)
        ws_seq, ws_start, ws_count = (np.array(x, dtype=np.int32) for x in (ws_seq, ws_start, ws_count))

        out = torch.empty((S, HQ, D), dtype=torch.bfloat16, device=dev)
        tab_dev = torch.from_numpy(np.ascontiguousarray(table[:S])).to(dev)
        kw = dict(scale=scale, max_context_len=int(L.max()), partition_size=partition, workspace=workspace)
        if pre is not None:
            row_slots = kv_build_slot_mapping(table[S:], B, N, np.zeros(1, np.int32), ws_start[S:], ws_count[S:])
            pool.paged_attention_decode_step(0, out, t16(q), t16(k_new), t16(v_new), tab_dev,
                                             torch.from_numpy(L).to(dev), t16(k_rows), t16(v_rows),
                                             torch.from_numpy(row_slots).to(dev), **kw)
            chunks += 1
        else:
            pool.paged_attention_decode_append(0, out, t16(q), t16(k_new), t16(v_new), tab_dev,
                                               torch.from_numpy(L).to(dev), **kw)
        torch.cuda.synchronize()

        slots = oracle.slot_mapping(table, B, N, ws_seq, ws_start, ws_count)
        if pre is not None:
            assert np.array_equal(row_slots, slots[S:]), f"step {step}: chunk slot mapping differs from the oracle's"
        kn = np.concatenate([k_new, k_rows])
        vn = np.concatenate([v_new, v_rows])
        if fp8:
            kc, vc, ks, vs = ofp8.scatter(kc, vc, ks, vs, kn, vn, slots, B)
            ref = ofp8.paged_attention(q, kc, vc, ks, vs, table[:S], L, scale)
        else:
            kp, vp = oracle.scatter(kp, vp, kn, vn, slots)
            ref = oracle.paged_attention(q, kp, vp, "bf16", table[:S], L, scale)
        got = to_f64(out.view(torch.int16).cpu().numpy().view(np.uint16), "bf16")
        assert np.isfinite(got).all(), f"step {step}: non-finite output (a NaN block was read)"
        err = float(np.abs(got - ref).max())
        worst = max(worst, err)
        assert err <= TOL["bf16"], f"step {step}: max |gpu - oracle| = {err:.3e}"

        if pre is not None:
            lens[pre] = c0 + n
            if lens[pre] == REQUESTS[pre][0]:
                batch.append(pre)           # its prompt is stored: it decodes from the next step on
        for r in list(batch):
            done = REQUESTS[r][3]
            if done is not None and step == done:
                batch.remove(r)
                for b in rows.pop(r):
                    alloc.release(b)
                    freed.add(b)

    say(f"  worst step: max |gpu - oracle| = {worst:.3e}; {chunks} prompt chunks, {reused} reused blocks")
    assert chunks >= 4 and reused > 0
    if fp8:
        for t, a in ((pool.k, kc), (pool.v, vc), (pool.k_scale, ks), (pool.v_scale, vs)):
            assert t.cpu().numpy().reshape(a.shape).tobytes() == a.tobytes(), "FP8 pool differs"
    else:
        gk = pool.k.view(torch.int16).cpu().numpy().view(np.uint16).reshape(kp.shape)
        gv = pool.v.view(torch.int16).cpu().numpy().view(np.uint16).reshape(vp.shape)
        assert gk.tobytes() == kp.tobytes() and gv.tobytes() == vp.tobytes(), "pool differs"
