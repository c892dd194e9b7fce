"""FP8 KV pools on the GPU (E4M3 codes, one fp32 scale per (block, KV head) for
K and one for V) against the oracle in oracle/fp8.py.

* Conversions: all 256 codes widened to bfloat16 (exact), and fp32 -> code
  rounding on every bfloat16 value, every tie between neighbouring codes and
  its neighbours, and random fp32 values: bit-exact.
* Scatter: codes and scales bit-exact for consecutive writes (blocks filled
  from row 0 in token order), a shuffled token order, writes continuing a
  block (stored scale, saturation), padding and out-of-pool slots, all-zero
  rows, on layer 1 of a two-layer pool (layer 0 untouched).
* Decode: the step (scatter of the decode rows, then attention) against the
  oracle's scatter and fp64 attention over the dequantized pool, within the
  bf16 tolerance, in the balanced, partitioned and single-workgroup modes,
  group sizes 1..8, edge lengths, NaN codes in every stale slot.
* Decode append: bitwise equal to the two-call step, and to the oracle.
* copy_blocks: codes and scales of every layer copied.
* The 8B-shaped batch (64 sequences, 512..4096 tokens): pool bit-exact,
  sampled sequences against the oracle.
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


@pytest.fixture(autouse=True)
def _need_gpu(gpu_available):
    yield


def _cuda(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


# ------------------------------------------------------------- conversions --

@pytest.mark.parametrize("shift", [0, 1, 2, 3])
def test_widen_all_codes_exactly(shift):
    """Each shift puts every code in the other byte of its pair and/or the other
    16-bit word of the operand, so both word selects are exercised per code."""
    import torch
    from paged_kv_cache_num_amd import probe_e4m3_to_bf16
    codes = np.roll(np.arange(256, dtype=np.uint8), shift)
    out = torch.empty(256, dtype=torch.int16, device="cuda")
    probe_e4m3_to_bf16(_cuda(codes), out)
    torch.cuda.synchronize()
    got = kvgen.bf16_bits_to_f32(out.cpu().numpy().view(np.uint16)).astype(np.float64)
    want = ofp8.e4m3_decode(codes)
    nan = np.isnan(want)
    assert nan.sum() == 2 and np.isnan(got[nan]).all()
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))   # -0 stays -0


def _encode_gpu(x):
    import torch
    from paged_kv_cache_num_amd import probe_f32_to_e4m3
    out = torch.empty(x.size, dtype=torch.uint8, device="cuda")
    probe_f32_to_e4m3(_cuda(x.astype(np.float32)), out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def test_encoder_matches_the_oracle_on_every_bf16_value_and_every_tie():
    every_bf16 = kvgen.bf16_bits_to_f32(np.arange(65536, dtype=np.uint16))   # zeros, subnormals, inf, NaN
    vals = ofp8.e4m3_decode(np.arange(0x7F, dtype=np.uint8))                  # the finite codes >= 0, increasing
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)                    # exact in fp32 (few bits)
    assert np.array_equal(mids.astype(np.float64), (vals[:-1] + vals[1:]) / 2)
    near = np.concatenate([mids, np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(0)),
                           vals.astype(np.float32)])
    edge = np.array([448.0, 448.00003, 464.0, 463.99997, 480.0, 1e30, 2.0**-10, 2.0**-9, 3 * 2.0**-10,
                     1e-45, 2.0**-6, np.nextafter(np.float32(2.0**-6), np.float32(0))], dtype=np.float32)
    x = np.concatenate([every_bf16, near, -near, edge, -edge])
    got = _encode_gpu(x)
    want = ofp8.e4m3_encode(x)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{bad.size} mismatches, e.g. x={x[bad[:5]]} gpu={got[bad[:5]]} oracle={want[bad[:5]]}"


def test_encoder_matches_the_oracle_on_random_fp32():
    rng = np.random.default_rng(81)
    n = 1 << 20
    mag = rng.uniform(1.0, 2.0, n) * np.exp2(rng.integers(-14, 11, n))
    x = (mag * rng.choice([-1.0, 1.0], n)).astype(np.float32)
    got = _encode_gpu(x)
    want = ofp8.e4m3_encode(x)
    assert np.array_equal(got, want), f"{int((got != want).sum())} mismatches"


# ----------------------------------------------------------------- scatter --

def _fp8_pool(layers, N, H, seed):
    from paged_kv_cache_num_amd import KVPool
    ss = np.random.SeedSequence([seed, 5])
    kc = kvgen.fp8_codes((N, H, 16, 128), ss.spawn(1)[0])
    vc = kvgen.fp8_codes((N, H, 16, 128), ss.spawn(1)[0])
    rng = np.random.default_rng(seed)
    ks = np.exp(rng.normal(math.log(4.0 / 448), 0.5, (N, H))).astype(np.float32)
    vs = np.exp(rng.normal(math.log(4.0 / 448), 0.5, (N, H))).astype(np.float32)
    pool = KVPool.allocate(num_layers=layers, num_blocks=N, block_size=16, num_kv_heads=H, head_dim=128,
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


SCATTER_CASES = ["runs", "shuffled", "zeros", "loud"]


@pytest.mark.parametrize("case", SCATTER_CASES)
def test_scatter_matches_the_oracle_bit_exactly(case):
    import torch
    say(f"fp8 scatter case={case}")
    N, H, B = 48, 8, 16
    pool, (kc, vc, ks, vs) = _fp8_pool(2, N, H, seed=3)
    rng = np.random.default_rng(17)
    tables = rng.permutation(N)[:40].astype(np.int32).reshape(4, 10)
    # seq 0 fills blocks 0, 1 and 5 rows of 2; seq 1 starts at block 1 (row 0) and ends
    # 2 rows into block 3; seq 2 continues block 0 at rows 5..8 (the stored scale);
    # seq 3 writes its block 4 whole
    ws, wst, wc = [0, 1, 2, 3], [0, 16, 5, 64], [37, 34, 4, 16]
    slots = oracle.slot_mapping(tables, B, N, ws, wst, wc)
    T = slots.size
    ss = np.random.SeedSequence([29, SCATTER_CASES.index(case)])
    kn = kvgen.normal_fill((T, H, 128), ss.spawn(1)[0], 1.0, "bf16")
    vn = kvgen.normal_fill((T, H, 128), ss.spawn(1)[0], 1.0, "bf16")
    if case == "zeros":
        kn[:16] = 0                     # block 0 of seq 0: K scale 1.0, codes 0
        vn[37:37 + 16] = 0x8000         # -0.0 everywhere in seq 1's first block
    if case == "loud":
        kn[71:75] = kvgen.f32_to_bf16_bits(kvgen.bf16_bits_to_f32(kn[71:75]) * 300.0)   # saturates
    # padding and an out-of-pool slot, mixed in
    slots = np.concatenate([slots[:20], [-1], slots[20:50], [N * B + 3], slots[50:]]).astype(np.int64)
    pad = np.zeros((1, H, 128), dtype=np.uint16)
    kn = np.concatenate([kn[:20], pad, kn[20:50], pad, kn[50:]])
    vn = np.concatenate([vn[:20], pad, vn[20:50], pad, vn[50:]])
    if case == "shuffled":
        perm = np.random.default_rng(5).permutation(slots.size)
        slots, kn, vn = slots[perm], kn[perm], vn[perm]
    pool.reshape_and_cache(1, _cuda(kn.view(np.int16)).view(torch.bfloat16),
                           _cuda(vn.view(np.int16)).view(torch.bfloat16), _cuda(slots))
    torch.cuda.synchronize()
    want = ofp8.scatter(kc, vc, ks, vs, kn, vn, slots, B)
    got = _host(pool, 1)
    for name, g, w in zip(("K codes", "V codes", "K scales", "V scales"), got, want):
        assert g.tobytes() == w.tobytes(), f"{case}: {name} differ at {np.argwhere(g != w)[:4].tolist()}"
    for g, w in zip(_host(pool, 0), (kc, vc, ks, vs)):
        assert g.tobytes() == w.tobytes(), "layer 0 must be untouched"
    if case == "zeros":
        assert got[2][tables[0, 0], :].tolist() == [1.0] * H


# ------------------------------------------------------------------ decode --

def _reference(wl, state, slots, scale):
    kc, vc, ks, vs = ofp8.scatter(*state, wl.k_new, wl.v_new, slots, wl.block_size)
    out = ofp8.paged_attention(wl.q, kc, vc, ks, vs, wl.block_tables, wl.context_lens, scale)
    return (kc, vc, ks, vs), out


def _check(step, wl, ref_pool, ref_out, label, check_pool=True):
    if check_pool:
        kc, vc = step.pool_host()
        ks, vs = step.scales_host()
        for name, g, w in zip(("K codes", "V codes", "K scales", "V scales"), (kc, vc, ks, vs), ref_pool):
            assert g.tobytes() == w.tobytes(), f"{label}: {name} differ"
    out = kvgen.bf16_bits_to_f32(step.out_host()).astype(np.float64)
    assert np.isfinite(out).all(), f"{label}: non-finite output"
    err = float(np.abs(out - ref_out).max()) if out.size else 0.0
    say(f"  {label}: max |gpu - oracle| = {err:.3e} (tol {TOL['bf16']:.0e})")
    assert err <= TOL["bf16"], f"{label}: error {err}"
    return err


DECODE = [
    ([1, 2, 15, 16, 17, 0, 33, 4096], 32, 8, 0),
    ([1, 16, 17, 300], 8, 8, 0),          # g = 1
    ([0, 31, 32, 3000], 16, 8, 0),        # g = 2
    ([5000, 20, 700, 1], 64, 8, 0),       # g = 8
    ([0, 7, 0, 1600, 2500], 32, 8, 512),  # partitions + merge
    ([100, 2000, 48], 32, 8, 64),
    ([3, 4000], 32, 8, 4096),             # one partition per sequence
]


@pytest.mark.parametrize("lengths,hq,hkv,partition", DECODE)
def test_decode_step_matches_the_oracle(lengths, hq, hkv, partition):
    import torch
    from paged_kv_cache_num_amd import DecodeStep
    say(f"fp8 decode lengths={lengths} Hq={hq} Hkv={hkv} partition={partition}")
    wl = kvgen.custom_workload(lengths=lengths, num_q_heads=hq, num_kv_heads=hkv, head_dim=128, dtype="bf16",
                               seed=41, variant="sharp", poison=True, table_pad=2)
    state = kvgen.fp8_pool_state(wl, seed=7)
    step = DecodeStep.from_workload(wl, fp8_pool=state, partition_size=partition)
    step.run()
    torch.cuda.synchronize()
    slots = oracle.slot_mapping(wl.all_tables(), wl.block_size, wl.num_blocks, wl.write_seq, wl.write_start,
                                wl.write_count)
    assert np.array_equal(step.slots_host, slots)
    ref_pool, ref_out = _reference(wl, state, slots, step.scale)
    _check(step, wl, ref_pool, ref_out, f"fp8 p{partition}")
    for i, L in enumerate(lengths):
        if L == 0:
            assert not kvgen.bf16_bits_to_f32(step.out_host()[i]).any()


def test_decode_wide_scale_spread_relative_error():
    """Block scales spread over e^(+-1.5): outputs reach ~20, where rounding the
    output to bfloat16 alone moves it by up to 20 * 2^-9.  Checked per output
    row relative to the row's magnitude (at least 1)."""
    import torch
    from paged_kv_cache_num_amd import DecodeStep
    wl = kvgen.custom_workload(lengths=[5000, 20, 700, 1], num_q_heads=64, num_kv_heads=8, head_dim=128,
                               dtype="bf16", seed=41, variant="sharp", poison=True, table_pad=2)
    state = kvgen.fp8_pool_state(wl, seed=7, largest=4.0, spread=0.5)
    step = DecodeStep.from_workload(wl, fp8_pool=state, partition_size=0)
    step.run()
    torch.cuda.synchronize()
    _, ref_out = _reference(wl, state, step.slots_host, step.scale)
    out = kvgen.bf16_bits_to_f32(step.out_host()).astype(np.float64)
    mag = np.maximum(1.0, np.abs(ref_out).max(axis=-1, keepdims=True))
    rel = float((np.abs(out - ref_out) / mag).max())
    say(f"  wide spread: max |gpu - oracle| / max(1, |row|) = {rel:.3e}, largest |out| {np.abs(ref_out).max():.2f}")
    assert rel <= TOL["bf16"]


def test_decode_more_sequences_than_the_balanced_split_takes():
    """1100 sequences: past the balanced split's batch limit, one workgroup per (sequence, KV head)."""
    import torch
    from paged_kv_cache_num_amd import DecodeStep
    lengths = np.random.default_rng(3).integers(1, 80, 1100)
    wl = kvgen.custom_workload(lengths=lengths, num_q_heads=8, num_kv_heads=2, head_dim=128, dtype="bf16",
                               seed=43, variant="sharp", poison=True)
    state = kvgen.fp8_pool_state(wl, seed=9)
    step = DecodeStep.from_workload(wl, fp8_pool=state, partition_size=0)
    assert step.workspace is None    # single-partition mode
    step.run()
    torch.cuda.synchronize()
    ref_pool, ref_out = _reference(wl, state, step.slots_host, step.scale)
    _check(step, wl, ref_pool, ref_out, "fp8 S=1100")


@pytest.mark.parametrize("lengths,hq,hkv,partition", DECODE[:5])
def test_decode_append_equals_two_calls_and_the_oracle(lengths, hq, hkv, partition):
    import torch
    from paged_kv_cache_num_amd import DecodeStep
    say(f"fp8 decode append lengths={lengths} partition={partition}")
    wl = kvgen.custom_workload(lengths=lengths, num_q_heads=hq, num_kv_heads=hkv, head_dim=128, dtype="bf16",
                               seed=47, variant="sharp", poison=True, table_pad=1)
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
    _check(fused, wl, ref_pool, ref_out, f"fp8 append p{partition}")


def test_decode_is_independent_of_block_placement():
    """The same logical contents under another block permutation: bitwise equal output."""
    import torch
    from paged_kv_cache_num_amd import DecodeStep
    wl = kvgen.custom_workload(lengths=[40, 1000, 17, 2500], num_q_heads=32, num_kv_heads=8, head_dim=128,
                               dtype="bf16", seed=53, variant="sharp", poison=False)
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


# ------------------------------------------------------------- copy blocks --

def test_copy_blocks_copies_codes_and_scales_of_every_layer():
    import torch
    layers, N, H = 3, 40, 8
    pool, (kc, vc, ks, vs) = _fp8_pool(layers, N, H, seed=19)
    pairs = np.array([[3, 30], [7, 8], [0, 39], [5, 45], [-1, 2], [11, 12]], dtype=np.int32)
    pool.copy_blocks(_cuda(pairs))
    torch.cuda.synchronize()
    stack = lambda a: np.stack([a] * layers)
    ek, ev = oracle.copy_blocks(stack(kc), stack(vc), pairs)
    eks, evs = oracle.copy_blocks(stack(ks)[..., None, None], stack(vs)[..., None, None], pairs)
    for li in range(layers):
        g = _host(pool, li)
        assert g[0].tobytes() == ek[li].tobytes() and g[1].tobytes() == ev[li].tobytes(), f"codes, layer {li}"
        assert g[2].tobytes() == eks[li, ..., 0, 0].tobytes() and g[3].tobytes() == evs[li, ..., 0, 0].tobytes()


# ------------------------------------------------- the 8B-shaped decode batch --

@pytest.mark.parametrize("variant", ["spec", "sharp"])
def test_8b_batch_pool_exact_and_every_sequence(variant):
    """The full 8B-shaped batch on an FP8 pool, the fused append in the
    balanced split (2048 workers): codes and scales bit-exact, and every one of
    the 64 sequences within 2e-2 of the FP8 oracle (each sequence's blocks
    gathered into a pool of their own, so the oracle runs one sequence at a time)."""
    import torch
    from paged_kv_cache_num_amd import DecodeStep
    say(f"C2 fp8 full batch, {variant}")
    wl = kvgen.make_workload("C2", variant=variant, poison=True)
    largest = 3.0 / math.sqrt(128) if variant == "spec" else 3.0
    state = kvgen.fp8_pool_state(wl, seed=2, largest=largest)
    step = DecodeStep.from_workload(wl, fp8_pool=state, partition_size=0)
    step.run_fused()
    torch.cuda.synchronize()
    ref = ofp8.scatter(*state, wl.k_new, wl.v_new, step.slots_host, wl.block_size)
    got = step.pool_host() + step.scales_host()
    for name, g, w in zip(("K codes", "V codes", "K scales", "V scales"), got, ref):
        assert g.tobytes() == w.tobytes(), f"C2 fp8: {name} differ"
    out = kvgen.bf16_bits_to_f32(step.out_host()).astype(np.float64)
    assert np.isfinite(out).all()
    B = wl.block_size
    worst = 0.0
    for i in range(wl.num_seqs):
        L = int(wl.context_lens[i])
        blocks = wl.block_tables[i, :-(-L // B)]
        sub = [a[blocks] for a in ref]
        want = ofp8.paged_attention(wl.q[i:i + 1], *sub, np.arange(blocks.size, dtype=np.int32)[None, :],
                                    np.array([L], dtype=np.int32), step.scale)
        worst = max(worst, float(np.abs(out[i] - want[0]).max()))
    say(f"  C2 fp8 {variant}, all {wl.num_seqs} sequences: max |gpu - oracle| = {worst:.3e}")
    assert worst <= TOL["bf16"]


@pytest.mark.parametrize("fused,partition", [(True, 0), (False, 512)])
def test_tp8_shard_one_kv_head_every_sequence(fused, partition):
    """One GPU's share of the 70B-class batch at TP = 8 (8 query heads, 1 KV
    head, 256 sequences, the 2048-token prefill chunk) on an FP8 pool: codes
    and scales bit-exact after the step, every sequence within 2e-2 of the
    FP8 oracle."""
    import torch
    from paged_kv_cache_num_amd import DecodeStep
    say(f"C3TP8 fp8 sharp, fused={fused}, partition={partition}")
    wl = kvgen.make_workload("C3TP8", variant="sharp", poison=True)
    state = kvgen.fp8_pool_state(wl, seed=3, largest=3.0)
    step = DecodeStep.from_workload(wl, fp8_pool=state, partition_size=partition)
    (step.run_fused if fused else step.run)()
    torch.cuda.synchronize()
    ref = ofp8.scatter(*state, wl.k_new, wl.v_new, step.slots_host, wl.block_size)
    for name, g, w in zip(("K codes", "V codes", "K scales", "V scales"), step.pool_host() + step.scales_host(), ref):
        assert g.tobytes() == w.tobytes(), f"C3TP8 fp8: {name} differ"
    want = ofp8.paged_attention(wl.q, *ref, wl.block_tables, wl.context_lens, step.scale)
    out = kvgen.bf16_bits_to_f32(step.out_host()).astype(np.float64)
    err = float(np.abs(out - want).max())
    say(f"  C3TP8 fp8: max |gpu - oracle| = {err:.3e}")
    assert np.isfinite(out).all() and err <= TOL["bf16"]


@pytest.mark.parametrize("fused,partition", [(False, 0), (True, 0), (False, 512), (True, 512)])
def test_graph_replays_match_eager_steps(fused, partition):
    """A captured FP8 step (scatter + attention, or the fused append) gives the
    eager step's output and pool bits on every replay, with eager work between
    the replays (the FP8 write path rewrites the same codes and scales each time)."""
    import torch
    from paged_kv_cache_num_amd import DecodeStep
    wl = kvgen.custom_workload(lengths=[700, 1, 16, 2049, 300, 33], num_q_heads=32, num_kv_heads=8, head_dim=128,
                               dtype="bf16", seed=67, variant="sharp", poison=True, table_pad=1)
    state = kvgen.fp8_pool_state(wl, seed=17)
    step = DecodeStep.from_workload(wl, fp8_pool=state, partition_size=partition)
    (step.run_fused if fused else step.run)()
    torch.cuda.synchronize()
    eager = step.out_host().copy()
    pool = [a.copy() for a in step.pool_host() + step.scales_host()]
    graph = step.capture(fused=fused)
    for i in range(4):
        step.out.fill_(0)
        junk = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        del junk
        assert np.array_equal(step.out_host(), eager), f"replay {i}: output differs from the eager step"
        for g, w in zip(step.pool_host() + step.scales_host(), pool):
            assert g.tobytes() == w.tobytes(), f"replay {i}: pool differs"


@pytest.mark.parametrize("S,partition", [(1024, 0), (1000, 64)])
def test_decode_at_the_balanced_split_batch_limit(S, partition):
    """1024 sequences (every chunk of the worker prologue's length scan) and a
    ragged 1000, on an FP8 pool: pool and outputs against the oracle."""
    import torch
    from paged_kv_cache_num_amd import DecodeStep
    say(f"fp8 S={S} partition={partition}")
    lengths = np.random.default_rng(S + 7).integers(0, 200, S)
    lengths[-1] = 199
    wl = kvgen.custom_workload(lengths=lengths, num_q_heads=16, num_kv_heads=4, head_dim=128, dtype="bf16",
                               seed=49, variant="sharp", poison=True)
    state = kvgen.fp8_pool_state(wl, seed=11)
    step = DecodeStep.from_workload(wl, fp8_pool=state, partition_size=partition)
    assert step.workspace is not None
    step.run()
    torch.cuda.synchronize()
    ref_pool, ref_out = _reference(wl, state, step.slots_host, step.scale)
    _check(step, wl, ref_pool, ref_out, f"fp8 S={S} p{partition}")
