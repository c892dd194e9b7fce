"""HIP path vs the CPU oracle on the GPU: scatter bit-exact, attention within
1e-4 (fp32) / 2e-2 (bf16), at the full configuration sizes and on edge cases.

Every case prints its name, seed and shape before it touches the GPU.
"""
import numpy as np
import pytest

import kvgen
import oracle
from parity_util import TOL, check_step, max_err, reference, run_gpu, say, to_f64, workload

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu(gpu_available):
    yield


# --------------------------------------------------------- full configs --

C1_CASES = [(v, p) for v in ("spec", "sharp", "hot", "needle") for p in (0, 32, 64)]


@pytest.mark.parametrize("variant,partition", C1_CASES)
def test_c1_tiny_fp32(variant, partition):
    say(f"C1 variant={variant} partition={partition}")
    wl = workload("C1", variant)
    ref = reference("C1", variant)
    step = run_gpu(wl, partition_size=partition)
    check_step(step, wl, ref, label=f"C1/{variant}/p{partition}")


@pytest.mark.parametrize("variant", ["spec", "sharp", "hot", "needle"])
@pytest.mark.parametrize("partition", [0, 512])
def test_c2_llama8b_decode(variant, partition):
    say(f"C2 variant={variant} partition={partition} S=64 Hq=32 Hkv=8 D=128 bf16")
    wl = workload("C2", variant)
    ref = reference("C2", variant)
    step = run_gpu(wl, partition_size=partition)
    check_step(step, wl, ref, label=f"C2/{variant}/p{partition}")


@pytest.mark.parametrize("variant", ["spec", "sharp", "needle"])
@pytest.mark.parametrize("partition", [0, 512])
def test_c3_70b_gqa8_with_prefill_scatter(variant, partition):
    say(f"C3 variant={variant} partition={partition} S=256 Hq=64 Hkv=8 D=128 bf16, 2048-token prefill chunk")
    wl = workload("C3", variant)
    ref = reference("C3", variant)
    step = run_gpu(wl, partition_size=partition)
    check_step(step, wl, ref, label=f"C3/{variant}/p{partition}")


@pytest.mark.parametrize("variant", ["spec", "sharp", "hot", "needle"])
@pytest.mark.parametrize("partition", [0, 512])
def test_c3_tp8_shard_one_kv_head(variant, partition):
    """One GPU's share of the 70B-class batch under tensor parallelism over KV
    heads at TP = 8 ("KV Cache & PagedAttention", section 5: each GPU holds
    H_kv / TP heads' cache): 8 query heads on 1 KV head, the same 256
    sequences and prefill chunk; the balanced split walks 256 (sequence, KV
    head) pairs over the whole GPU."""
    say(f"C3TP8 variant={variant} partition={partition} S=256 Hq=8 Hkv=1 D=128 bf16, 2048-token prefill chunk")
    wl = workload("C3TP8", variant)
    ref = reference("C3TP8", variant)
    step = run_gpu(wl, partition_size=partition)
    check_step(step, wl, ref, label=f"C3TP8/{variant}/p{partition}")


@pytest.mark.parametrize("partition", [0, 512])
def test_c4_prefix_sharing_equals_private_copies(partition):
    say(f"C4 sharp S=128 shared 2048-token prefix, partition={partition}")
    wl = workload("C4", "sharp")
    ref = reference("C4", "sharp")
    shared = run_gpu(wl, partition_size=partition)
    check_step(shared, wl, ref, label=f"C4/shared/p{partition}")
    priv = kvgen.privatize_blocks(wl)
    say("C4 private copies")
    private = run_gpu(priv, partition_size=partition)
    assert np.array_equal(shared.out_host(), private.out_host()), "shared and private copies differ"


@pytest.mark.parametrize("variant", ["sharp", "needle"])
@pytest.mark.parametrize("partition", [512, 0])
def test_c5_long_context_split(variant, partition):
    say(f"C5 variant={variant} S=8 L in [32768,131072] partition={partition}")
    wl = workload("C5", variant)
    ref = reference("C5", variant)
    step = run_gpu(wl, partition_size=partition)
    check_step(step, wl, ref, label=f"C5/{variant}/p{partition}")


# ------------------------------------------------------------ invariances --

@pytest.mark.parametrize("partition", [0, 512])
def test_bitwise_invariance_to_block_placement(partition):
    say(f"C2 sharp: permuted and contiguous placements, partition={partition}")
    wl = workload("C2", "sharp")
    base = run_gpu(wl, partition_size=partition).out_host()
    for seed in (1, 2):
        perm = run_gpu(kvgen.permute_blocks(wl, seed), partition_size=partition).out_host()
        assert np.array_equal(base, perm), f"permutation {seed} changed the output bits"
    dense = run_gpu(kvgen.privatize_blocks(wl, contiguous=True), partition_size=partition).out_host()
    assert np.array_equal(base, dense), "identity (contiguous) tables changed the output bits"


def test_repeated_runs_are_bitwise_identical():
    import torch
    say("C2 sharp: repeated runs")
    wl = workload("C2", "sharp")
    step = run_gpu(wl, partition_size=512)
    first = step.out_host()
    for _ in range(3):
        step.attend()
        torch.cuda.synchronize()
        assert np.array_equal(first, step.out_host())


@pytest.mark.parametrize("name,partition", [("C2", 0), ("C2", 512), ("C3", 0), ("C1", 32)])
def test_graph_replays_match_eager_calls(name, partition):
    """A captured step gives the eager step's bits on every replay, with eager
    work (a fill of the output, a reduction) between the replays."""
    import torch
    say(f"{name} sharp: HIP graph capture of the step, partition={partition}")
    wl = workload(name, "sharp")
    step = run_gpu(wl, partition_size=partition)
    eager = step.out_host()
    graph = step.capture()
    for i in range(4):
        step.out.fill_(0)
        junk = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        del junk
        assert np.array_equal(step.out_host(), eager), f"replay {i} differs from the eager call"


@pytest.mark.parametrize("partition", [16, 48, 128, 1024, 4096])
def test_partition_sizes_agree_with_the_oracle(partition):
    say(f"C2 sharp partition={partition}")
    wl = workload("C2", "sharp")
    ref = reference("C2", "sharp")
    step = run_gpu(wl, partition_size=partition)
    check_step(step, wl, ref, check_pool=False, label=f"C2/p{partition}")


# ------------------------------------------------------------- edge cases --

EDGE = [
    # (dtype, Hq, Hkv, D, lengths, partition)
    ("bf16", 8, 8, 128, [1, 2, 15, 16, 17], 0),         # g = 1
    ("bf16", 16, 8, 128, [33, 64, 65, 1000], 64),       # g = 2
    ("bf16", 64, 8, 64, [300, 5, 129], 0),              # g = 8, D = 64
    ("bf16", 32, 8, 64, [511, 512, 513, 2048], 512),    # partition edges, D = 64
    ("f32", 8, 2, 128, [17, 1, 250, 3000], 256),        # fp32, D = 128
    ("f32", 16, 2, 64, [4096, 31], 0),                  # fp32, g = 8
    ("bf16", 32, 8, 128, [0, 7, 0, 40], 0),             # empty sequences
    ("bf16", 32, 8, 128, [0, 7, 0, 1600], 512),         # empty sequences, split
    ("bf16", 64, 8, 128, [0, 0, 0], 0),                 # nothing to attend to at all
    ("bf16", 8, 8, 128, [1], 0),                        # fewer tiles than workers
    ("bf16", 16, 8, 128, [3000, 1, 0, 17, 4096, 33], 0),  # ragged, balanced split, g = 2
    ("bf16", 64, 8, 128, [5000, 20, 700], 0),           # g = 8, balanced split
    ("bf16", 16, 8, 128, [1, 2, 15, 16, 17], 0),        # fewer tiles than workers, split pairs (g = 2)
    ("bf16", 8, 8, 128, [40, 300], 0),                  # fewer tiles than workers, split pairs (g = 1)
]


@pytest.mark.parametrize("dtype,hq,hkv,d,lengths,partition", EDGE)
def test_edge_shapes(dtype, hq, hkv, d, lengths, partition):
    say(f"edge dtype={dtype} Hq={hq} Hkv={hkv} D={d} lengths={lengths} partition={partition}")
    for variant in ("sharp", "hot"):
        wl = kvgen.custom_workload(lengths=lengths, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                                   dtype=dtype, seed=21, variant=variant, poison=True, table_pad=3)
        ref = oracle.run_step(wl)
        step = run_gpu(wl, partition_size=partition)
        check_step(step, wl, ref, label=f"edge/{variant}")
        for i, L in enumerate(lengths):
            if L == 0:
                assert not to_f64(step.out_host()[i], dtype).any(), "zero-length sequence must give zeros"


def test_single_token_output_is_its_value_bit_exact():
    say("single-token contexts: out == v_new bits")
    for dtype in ("bf16", "f32"):
        wl = kvgen.custom_workload(lengths=[1, 1, 1, 1], num_q_heads=8, num_kv_heads=2, head_dim=128,
                                   dtype=dtype, seed=4, variant="hot", poison=True)
        step = run_gpu(wl)
        out = step.out_host()
        for i in range(4):
            for h in range(8):
                assert out[i, h].tobytes() == wl.v_new[i, h // 4].tobytes()


def test_other_layer_of_a_multi_layer_pool():
    import torch
    say("3-layer pool, layer 1")
    wl = kvgen.custom_workload(lengths=[100, 37, 260], num_q_heads=32, num_kv_heads=8, head_dim=128,
                               dtype="bf16", seed=8, variant="sharp", poison=True)
    ref = oracle.run_step(wl)
    step = run_gpu(wl, num_layers=3, layer=1, partition_size=64)
    check_step(step, wl, ref, label="layer 1 of 3")
    k0, _ = step.pool_host(layer=0)
    k2, _ = step.pool_host(layer=2)
    assert k0.tobytes() == wl.k_pool.tobytes() and k2.tobytes() == wl.k_pool.tobytes(), \
        "scatter wrote outside its layer"


def test_padding_tokens_with_negative_slots_are_skipped():
    import torch
    say("scatter with padding slots")
    wl = workload("C1", "sharp")
    step = run_gpu(wl)
    kp0, vp0 = step.pool_host()
    pad = torch.full((4,), -1, dtype=torch.int64, device="cuda")
    step.pool.reshape_and_cache(0, step.k_new, step.v_new, pad)
    torch.cuda.synchronize()
    kp1, vp1 = step.pool_host()
    assert kp0.tobytes() == kp1.tobytes() and vp0.tobytes() == vp1.tobytes()


@pytest.mark.parametrize("name,variant,num_seqs", [("C2", "sharp", None), ("C3", "needle", 96), ("C5", "sharp", None)])
def test_balanced_merge_reads_fresh_partial_states(name, variant, num_seqs):
    """Split (sequence, KV head) pairs are merged from this call's partial states.

    Between calls every workspace byte is overwritten with NaN patterns by a
    separate kernel; each later call must still match the oracle.
    """
    import torch
    say(f"{name} {variant} balanced split, workspace poisoned between calls")
    wl = kvgen.make_workload(name, variant=variant, poison=True, num_seqs=num_seqs)
    ref = oracle.run_step(wl)
    step = run_gpu(wl, partition_size=0)
    check_step(step, wl, ref, check_pool=False, label=f"{name}/first call")
    for _ in range(2):
        step.workspace.fill_(0xFF)
        step.out.fill_(0)
        step.attend()
        torch.cuda.synchronize()
        err = max_err(step.out_host(), ref["out"], wl.dtype)
        say(f"  after poisoning: max err {err:.3e}")
        assert err <= TOL[wl.dtype]


@pytest.mark.parametrize("T", [2051, 4099])
def test_large_ragged_scatter_bit_exact(T):
    """reshape_and_cache with thousands of rows (the kernel then moves four
    tokens per workgroup) and a count that is not a multiple of four, with
    padding slots (-1) and slots past the pool mixed in: the pool equals the
    oracle's scatter of the in-range rows, byte for byte."""
    import torch
    from paged_kv_cache_num_amd.kvpool import KVPool
    from paged_kv_cache_num_amd.step import to_device, to_host
    N, H, B, D = 700, 8, 16, 128
    say(f"scatter of {T} rows into an [{N}][{H}][{B}][{D}] bf16 pool, padding and out-of-range slots")
    rng = np.random.default_rng(T)
    kp = rng.integers(0, 1 << 16, size=(N, H, B, D), dtype=np.uint16)
    vp = rng.integers(0, 1 << 16, size=(N, H, B, D), dtype=np.uint16)
    kn = rng.integers(0, 1 << 16, size=(T, H, D), dtype=np.uint16)
    vn = rng.integers(0, 1 << 16, size=(T, H, D), dtype=np.uint16)
    slots = rng.permutation(N * B)[:T].astype(np.int64)
    slots[::7] = -1
    slots[5::97] = N * B + 3
    keep = (slots >= 0) & (slots < N * B)
    want_k, want_v = oracle.scatter(kp, vp, kn[keep], vn[keep], slots[keep])
    pool = KVPool(to_device(kp, "bf16"), to_device(vp, "bf16"), num_layers=1, num_blocks=N, block_size=B,
                  num_kv_heads=H, head_dim=D)
    pool.reshape_and_cache(0, to_device(kn, "bf16"), to_device(vn, "bf16"),
                           torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    assert to_host(pool.k, "bf16").tobytes() == want_k.tobytes()
    assert to_host(pool.v, "bf16").tobytes() == want_v.tobytes()


# The fix-up gives each wave GH of a (sequence, KV head) pair's G query heads,
# GH halved from G while the grid would hold fewer than 1024 waves.  One case
# per (G, GH) the host can pick, with lengths that split every walk over
# several workers' records: (Hq, Hkv, sequences, GH expected).
FIXUP_SPLITS = [
    (8, 8, 16, 1),      # G = 1
    (16, 8, 32, 1),     # G = 2: 256 pairs
    (16, 8, 128, 2),    #        1024 pairs
    (32, 8, 16, 1),     # G = 4: 128 pairs
    (32, 8, 64, 2),     #        512 pairs
    (32, 8, 128, 4),    #        1024 pairs
    (64, 8, 8, 1),      # G = 8: 64 pairs
    (64, 8, 32, 2),     #        256 pairs
    (64, 8, 64, 4),     #        512 pairs
    (64, 8, 128, 8),    #        1024 pairs
]


@pytest.mark.parametrize("hq,hkv,num_seqs,gh", FIXUP_SPLITS)
def test_fixup_heads_per_wave(hq, hkv, num_seqs, gh):
    g = hq // hkv
    pairs = num_seqs * hkv
    expect = g
    while expect > 1 and pairs * (g // expect) < 1024:
        expect //= 2
    assert expect == gh, "the case no longer hits the heads-per-wave it is meant for"
    rng = np.random.default_rng(1000 + 10 * g + num_seqs)
    lengths = rng.integers(16, 1200, size=num_seqs).astype(np.int32)
    lengths[0] = 1   # a single-token walk among the split ones
    say(f"fix-up G={g} GH={gh}: Hq={hq} Hkv={hkv} S={num_seqs} lengths {int(lengths.min())}..{int(lengths.max())}")
    for variant in ("sharp", "hot"):
        wl = kvgen.custom_workload(lengths=lengths, num_q_heads=hq, num_kv_heads=hkv, head_dim=128,
                                   dtype="bf16", seed=31 + g, variant=variant, poison=True)
        ref = oracle.run_step(wl)
        step = run_gpu(wl, partition_size=0)
        check_step(step, wl, ref, check_pool=False, label=f"fix-up G={g} GH={gh}/{variant}")


# The balanced split's batch limit: the worker prologue loads the lengths of
# up to 16 chunks of 64 sequences at once and scans them chunk by chunk; the
# partitions kernel does the same.  1024 sequences fill every chunk, 1000
# leave the last one ragged, 65 put one sequence in a second chunk.
@pytest.mark.parametrize("S,partition", [(1024, 0), (1000, 0), (65, 0), (1024, 64), (1000, 128)])
def test_batch_size_up_to_the_balanced_split_limit(S, partition):
    say(f"bf16 S={S} partition={partition}: every chunk of the length scan")
    lengths = np.random.default_rng(S + partition).integers(0, 300, S)
    lengths[-1] = 299   # the last sequence of the last chunk holds tiles
    wl = kvgen.custom_workload(lengths=lengths, num_q_heads=16, num_kv_heads=4, head_dim=128, dtype="bf16",
                               seed=47, variant="sharp", poison=True)
    ref = oracle.run_step(wl)
    step = run_gpu(wl, partition_size=partition)
    assert step.workspace is not None   # the balanced split or the partitions on its workers
    check_step(step, wl, ref, label=f"S={S} p{partition}")
