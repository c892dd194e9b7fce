"""FP8 pools at block sizes 8, 32, 64 and 128 (block size 16 is covered by
test_fp8_gpu.py) against the oracle in oracle/fp8.py.

* Scatter: codes and scales bit-exact for a prefill chunk that fills blocks
  whole (the scale is the amax over every row the call puts into a block, up
  to 128 rows) and leaves one partly filled, decode rows that open a block
  alone, rows continuing a block (its stored scale), in token order and
  shuffled (the scale kernel's search for a block's writers), with padding
  and an out-of-pool slot; layer 0 of the two-layer pool stays untouched.
* Decode step (scatter of the decode rows, then attention) in the balanced,
  partitioned and single-pass modes, G = 1, 4 and 8, lengths at block and
  tile edges (rows that open blocks), NaN codes in every stale slot: within
  the bf16 tolerance of fp64 attention over the dequantized pool.
* Decode append: bitwise equal to the two-call step and to the oracle,
  including new rows that open a block; with 8-token blocks, rows in either
  half of a 16-token tile (the tile spans two blocks with two scales).
* Placement: the same contents under another block permutation give bitwise
  the same output.
"""
import dataclasses
import math

import numpy as np
import pytest

import kvgen
import oracle
import oracle.fp8 as ofp8
from parity_util import TOL, say

pytestmark = pytest.mark.gpu

BLOCK_SIZES = [8, 32, 64, 128]


@pytest.fixture(autouse=True)
def _need_gpu(gpu_available):
    yield


def _cuda(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _fp8_pool(layers, N, H, B, seed):
    from paged_kv_cache_num_amd import KVPool
    ss = np.random.SeedSequence([seed, 5, B])
    kc = kvgen.fp8_codes((N, H, B, 128), ss.spawn(1)[0])
    vc = kvgen.fp8_codes((N, H, B, 128), ss.spawn(1)[0])
    rng = np.random.default_rng([seed, B])
    ks = np.exp(rng.normal(math.log(4.0 / 448), 0.5, (N, H))).astype(np.float32)
    vs = np.exp(rng.normal(math.log(4.0 / 448), 0.5, (N, H))).astype(np.float32)
    pool = KVPool.allocate(num_layers=layers, num_blocks=N, block_size=B, num_kv_heads=H, head_dim=128,
                           dtype="fp8", device="cuda")
    for li in range(layers):
        pool.k[li].copy_(_cuda(kc))
        pool.v[li].copy_(_cuda(vc))
        pool.k_scale[li].copy_(_cuda(ks))
        pool.v_scale[li].copy_(_cuda(vs))
    return pool, (kc, vc, ks, vs)


def _host(pool, li):
    return (pool.k[li].cpu().numpy(), pool.v[li].cpu().numpy(), pool.k_scale[li].cpu().numpy(),
            pool.v_scale[li].cpu().numpy())


@pytest.mark.parametrize("shuffled", [False, True])
@pytest.mark.parametrize("B", BLOCK_SIZES)
def test_scatter_matches_the_oracle_bit_exactly(B, shuffled):
    import torch
    say(f"fp8 scatter B={B} shuffled={shuffled}")
    N, H = 40, 4
    pool, (kc, vc, ks, vs) = _fp8_pool(2, N, H, B, seed=3)
    tables = np.random.default_rng([17, B]).permutation(N)[:32].astype(np.int32).reshape(4, 8)
    # seq 0: a prefill chunk over blocks 0 and 1 whole and rows 0..4 of block 2;
    # seq 1: one row at position B, opening its block 1 alone;
    # seq 2: rows 3 .. B+2, continuing block 0 (stored scale) and opening block 1;
    # seq 3: one row at position 0
    ws, wst, wc = [0, 1, 2, 3], [0, B, 3, 0], [2 * B + 5, 1, B, 1]
    slots = oracle.slot_mapping(tables, B, N, ws, wst, wc)
    T = slots.size
    ss = np.random.SeedSequence([29, B])
    kn = kvgen.normal_fill((T, H, 128), ss.spawn(1)[0], 1.0, "bf16")
    vn = kvgen.normal_fill((T, H, 128), ss.spawn(1)[0], 1.0, "bf16")
    # one loud row deep inside the prefill's first block: the block's scale must cover it
    kn[B - 1] = kvgen.f32_to_bf16_bits(kvgen.bf16_bits_to_f32(kn[B - 1]) * 40.0)
    slots = np.concatenate([slots[:7], [-1], slots[7:], [N * B + 3]]).astype(np.int64)
    pad = np.zeros((1, H, 128), dtype=np.uint16)
    kn = np.concatenate([kn[:7], pad, kn[7:], pad])
    vn = np.concatenate([vn[:7], pad, vn[7:], pad])
    if shuffled:
        perm = np.random.default_rng(5).permutation(slots.size)
        slots, kn, vn = slots[perm], kn[perm], vn[perm]
    pool.reshape_and_cache(1, _cuda(kn.view(np.int16)).view(torch.bfloat16),
                           _cuda(vn.view(np.int16)).view(torch.bfloat16), _cuda(slots))
    torch.cuda.synchronize()
    want = ofp8.scatter(kc, vc, ks, vs, kn, vn, slots, B)
    got = _host(pool, 1)
    for name, g, w in zip(("K codes", "V codes", "K scales", "V scales"), got, want):
        assert g.tobytes() == w.tobytes(), f"B={B}: {name} differ at {np.argwhere(g != w)[:4].tolist()}"
    for g, w in zip(_host(pool, 0), (kc, vc, ks, vs)):
        assert g.tobytes() == w.tobytes(), "layer 0 must be untouched"
    # the prefill's first block took its scale from all B of its rows, the loud one included
    assert np.all(got[2][tables[0, 0]] >= 30.0 / 448)


# ------------------------------------------------------------------ decode --

def _lengths(B):
    # L - 1 at row 0 of a block (opens it), at row 8 of a tile, mid-block, long
    return [1, B + 1, 2 * B + 1, 13, 0, 3 * B + 7, 1200, 2500]


def _reference(wl, state, slots, scale):
    kc, vc, ks, vs = ofp8.scatter(*state, wl.k_new, wl.v_new, slots, wl.block_size)
    out = ofp8.paged_attention(wl.q, kc, vc, ks, vs, wl.block_tables, wl.context_lens, scale)
    return (kc, vc, ks, vs), out


def _check(step, ref_pool, ref_out, label):
    kc, vc = step.pool_host()
    ks, vs = step.scales_host()
    for name, g, w in zip(("K codes", "V codes", "K scales", "V scales"), (kc, vc, ks, vs), ref_pool):
        assert g.tobytes() == w.tobytes(), f"{label}: {name} differ"
    out = kvgen.bf16_bits_to_f32(step.out_host()).astype(np.float64)
    assert np.isfinite(out).all(), f"{label}: non-finite output"
    err = float(np.abs(out - ref_out).max())
    say(f"  {label}: max |gpu - oracle| = {err:.3e} (tol {TOL['bf16']:.0e})")
    assert err <= TOL["bf16"], f"{label}: error {err}"


@pytest.mark.parametrize("hq", [8, 32, 64])
@pytest.mark.parametrize("partition", [0, 256, 4096])
@pytest.mark.parametrize("B", BLOCK_SIZES)
def test_decode_step_matches_the_oracle(B, partition, hq):
    import torch
    from paged_kv_cache_num_amd import DecodeStep
    say(f"fp8 decode B={B} partition={partition} Hq={hq}")
    lengths = _lengths(B)
    wl = kvgen.custom_workload(lengths=lengths, num_q_heads=hq, num_kv_heads=8, head_dim=128, dtype="bf16",
                               block_size=B, seed=41 + B, variant="sharp", poison=True, table_pad=2)
    state = kvgen.fp8_pool_state(wl, seed=7)
    step = DecodeStep.from_workload(wl, fp8_pool=state, partition_size=partition)
    step.run()
    torch.cuda.synchronize()
    slots = oracle.slot_mapping(wl.all_tables(), B, wl.num_blocks, wl.write_seq, wl.write_start, wl.write_count)
    assert np.array_equal(step.slots_host, slots)
    ref_pool, ref_out = _reference(wl, state, slots, step.scale)
    _check(step, ref_pool, ref_out, f"fp8 B={B} p{partition} Hq={hq}")
    assert not kvgen.bf16_bits_to_f32(step.out_host()[lengths.index(0)]).any()


@pytest.mark.parametrize("partition", [0, 256])
@pytest.mark.parametrize("B", BLOCK_SIZES)
def test_decode_append_equals_two_calls_and_the_oracle(B, partition):
    import torch
    from paged_kv_cache_num_amd import DecodeStep
    say(f"fp8 decode append B={B} partition={partition}")
    wl = kvgen.custom_workload(lengths=_lengths(B), num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16",
                               block_size=B, seed=47 + B, variant="sharp", poison=True, table_pad=1)
    state = kvgen.fp8_pool_state(wl, seed=11)
    two = DecodeStep.from_workload(wl, fp8_pool=state, partition_size=partition)
    fused = DecodeStep.from_workload(wl, fp8_pool=state, partition_size=partition)
    assert fused.can_fuse
    two.run()
    fused.run_fused()
    torch.cuda.synchronize()
    assert fused.out_host().tobytes() == two.out_host().tobytes()
    for a, b in zip(fused.pool_host() + fused.scales_host(), two.pool_host() + two.scales_host()):
        assert a.tobytes() == b.tobytes()
    ref_pool, ref_out = _reference(wl, state, two.slots_host, two.scale)
    _check(fused, ref_pool, ref_out, f"fp8 append B={B} p{partition}")


@pytest.mark.parametrize("B", [8, 64])
def test_decode_is_independent_of_block_placement(B):
    import torch
    from paged_kv_cache_num_amd import DecodeStep
    wl = kvgen.custom_workload(lengths=[40, 1000, 17, 2500], num_q_heads=32, num_kv_heads=8, head_dim=128,
                               dtype="bf16", block_size=B, seed=53, variant="sharp", poison=False)
    kc, vc, ks, vs = kvgen.fp8_pool_state(wl, seed=13)
    perm = np.random.default_rng(2).permutation(wl.num_blocks)     # new block p holds old block perm[p]
    inv = np.argsort(perm)                                          # old block b is new block inv[b]
    assert wl.extra_tables.size == 0
    wl2 = dataclasses.replace(wl, block_tables=inv[wl.block_tables].astype(np.int32))
    outs = []
    for w, st in ((wl, (kc, vc, ks, vs)), (wl2, (kc[perm], vc[perm], ks[perm], vs[perm]))):
        step = DecodeStep.from_workload(w, fp8_pool=st, partition_size=0)
        step.run()
        torch.cuda.synchronize()
        outs.append(step.out_host())
    assert outs[0].tobytes() == outs[1].tobytes()


# --------------------------------------------- the step with other rows --

@pytest.mark.parametrize("shuffled", [False, True])
@pytest.mark.parametrize("B", [8, 16, 32, 64, 128])
def test_step_rows_bitwise_the_scatter_then_the_append(B, shuffled):
    """paged_attention_decode_step on an FP8 pool stores the other rows from
    extra waves of the attention's launch, with the block scale rule: the rows
    of the scatter test above (a prefill chunk over two whole blocks and part
    of a third, with a loud row; a row opening a block alone; rows continuing a
    block with its stored scale and opening the next; a padding row and an
    out-of-pool slot; in token order or shuffled, which sends the writers'
    search through the whole mapping) beside a decode batch on other blocks.
    Codes, scales and output are bitwise those of reshape_and_cache followed
    by paged_attention_decode_append; the pool is the oracle's scatter of the
    rows and the appended rows; the output is within 2e-2 of the oracle."""
    import torch
    say(f"fp8 step with other rows B={B} shuffled={shuffled}")
    N, H, Hq = 80, 4, 16
    pool_a, state = _fp8_pool(2, N, H, B, seed=7)
    pool_b, _ = _fp8_pool(2, N, H, B, seed=7)
    perm = np.random.default_rng([23, B]).permutation(N).astype(np.int32)
    row_tables, dec_tables = perm[:32].reshape(4, 8), perm[32:64].reshape(4, 8)
    ws, wst, wc = [0, 1, 2, 3], [0, B, 3, 0], [2 * B + 5, 1, B, 1]
    slots = oracle.slot_mapping(row_tables, B, N, ws, wst, wc)
    T = slots.size
    ss = np.random.SeedSequence([31, B])
    kn = kvgen.normal_fill((T, H, 128), ss.spawn(1)[0], 1.0, "bf16")
    vn = kvgen.normal_fill((T, H, 128), ss.spawn(1)[0], 1.0, "bf16")
    kn[B - 1] = kvgen.f32_to_bf16_bits(kvgen.bf16_bits_to_f32(kn[B - 1]) * 40.0)
    slots = np.concatenate([slots[:7], [-1], slots[7:], [N * B + 3]]).astype(np.int64)
    pad = np.zeros((1, H, 128), dtype=np.uint16)
    kn = np.concatenate([kn[:7], pad, kn[7:], pad])
    vn = np.concatenate([vn[:7], pad, vn[7:], pad])
    if shuffled:
        p = np.random.default_rng(6).permutation(slots.size)
        slots, kn, vn = slots[p], kn[p], vn[p]
    # the decode batch: last positions at row 0 of a block, inside one, at a block's end
    lens = np.array([1, B + 1, 3 * B, 5 * B + 3], dtype=np.int32)
    S = lens.size
    q = kvgen.normal_fill((S, Hq, 128), ss.spawn(1)[0], 1.0, "bf16")
    ka = kvgen.normal_fill((S, H, 128), ss.spawn(1)[0], 1.0, "bf16")
    va = kvgen.normal_fill((S, H, 128), ss.spawn(1)[0], 1.0, "bf16")
    bf = lambda a: _cuda(a.view(np.int16)).view(torch.bfloat16)
    scale = 1.0 / math.sqrt(128)
    outs = []
    for pool, fused in ((pool_a, True), (pool_b, False)):
        ws_bytes = pool.workspace_bytes(S, Hq, int(lens.max()), 0)
        work = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
        out = torch.zeros((S, Hq, 128), dtype=torch.bfloat16, device="cuda")
        args = dict(scale=scale, max_context_len=int(lens.max()), partition_size=0, workspace=work)
        if fused:
            pool.paged_attention_decode_step(1, out, bf(q), bf(ka), bf(va), _cuda(dec_tables), _cuda(lens),
                                             bf(kn), bf(vn), _cuda(slots), **args)
        else:
            pool.reshape_and_cache(1, bf(kn), bf(vn), _cuda(slots))
            pool.paged_attention_decode_append(1, out, bf(q), bf(ka), bf(va), _cuda(dec_tables), _cuda(lens), **args)
        torch.cuda.synchronize()
        outs.append(out.view(torch.int16).cpu().numpy())
    assert outs[0].tobytes() == outs[1].tobytes(), "output differs from the two-call step"
    for li in (0, 1):
        for name, g, w in zip(("K codes", "V codes", "K scales", "V scales"), _host(pool_a, li), _host(pool_b, li)):
            assert g.tobytes() == w.tobytes(), f"B={B} layer {li}: {name} differ from the two-call step"
    app_slots = oracle.slot_mapping(dec_tables, B, N, list(range(S)), list(lens - 1), [1] * S)
    want = ofp8.scatter(*ofp8.scatter(*state, kn, vn, slots, B), ka, va, app_slots, B)
    for name, g, w in zip(("K codes", "V codes", "K scales", "V scales"), _host(pool_a, 1), want):
        assert g.tobytes() == w.tobytes(), f"B={B}: {name} differ from the oracle's scatter"
    ref = ofp8.paged_attention(q, *want, dec_tables, lens, scale)
    got = kvgen.bf16_bits_to_f32(outs[0].view(np.uint16)).astype(np.float64)
    err = float(np.abs(got - ref).max())
    say(f"  B={B} shuffled={shuffled}: max |gpu - oracle| = {err:.3e}")
    assert np.isfinite(got).all() and err <= TOL["bf16"]
