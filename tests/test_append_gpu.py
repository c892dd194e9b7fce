"""Decode append folded into the attention call (paged_attention_decode_append).

The fused step must give, bit for bit, the output and the pool of the two-call
step (reshape_and_cache of each sequence's new row at position L_i - 1, then
paged_attention_decode), and match the oracle within the dtype's tolerance.
Covered: the balanced mode (where the wave reading each last block writes the
row), the fixed-partition and fp32 / D = 64 modes (a scatter kernel first),
prefix-shared blocks, steps with a prefill chunk of another sequence stored in
the same call (paged_attention_decode_step), and edge lengths.
"""
import numpy as np
import pytest

import kvgen
import oracle
from parity_util import TOL, check_step, max_err, reference, say, to_f64, workload

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu(gpu_available):
    yield


def _both(wl, **kw):
    import torch
    from paged_kv_cache_num_amd import DecodeStep
    two = DecodeStep.from_workload(wl, **kw)
    two.run()
    fused = DecodeStep.from_workload(wl, **kw)
    assert fused.can_fuse
    fused.run_fused()
    torch.cuda.synchronize()
    return two, fused


def _same(two, fused, label):
    assert fused.out_host().tobytes() == two.out_host().tobytes(), f"{label}: output differs from the two-call step"
    k2, v2 = two.pool_host()
    kf, vf = fused.pool_host()
    assert kf.tobytes() == k2.tobytes() and vf.tobytes() == v2.tobytes(), f"{label}: pool differs"


# C3 and its TP-8 shard carry a 2048-token prefill chunk of a sequence outside
# the batch: the fused step stores it in the same call (paged_attention_decode_step;
# balanced mode: extra waves of the attention's launch, partitions: the scatter kernel first)
CASES = [("C1", "sharp", 0), ("C1", "hot", 32), ("C2", "spec", 0), ("C2", "needle", 0), ("C2", "sharp", 512),
         ("C3", "needle", 0), ("C3", "sharp", 512), ("C3TP8", "spec", 0), ("C4", "sharp", 0), ("C5", "needle", 0),
         ("C5", "sharp", 512)]


@pytest.mark.parametrize("name,variant,partition", CASES)
def test_fused_step_equals_two_calls_and_oracle(name, variant, partition):
    say(f"{name} {variant} partition={partition}: fused append vs two calls")
    wl = workload(name, variant)
    ref = reference(name, variant)
    two, fused = _both(wl, partition_size=partition)
    _same(two, fused, f"{name}/{variant}/p{partition}")
    check_step(fused, wl, ref, label=f"{name}/{variant}/p{partition} fused")


EDGE = [
    ("bf16", 32, 8, 128, [1, 2, 15, 16, 17, 0, 33, 4096], 0),
    ("bf16", 8, 8, 128, [1, 16, 17, 300], 0),        # g = 1
    ("bf16", 16, 8, 128, [0, 31, 32, 3000], 0),      # g = 2
    ("bf16", 64, 8, 128, [5000, 20, 700, 1], 0),     # g = 8
    ("bf16", 32, 8, 128, [0, 7, 0, 1600], 512),      # fixed partitions
    ("bf16", 32, 8, 64, [511, 512, 513], 0),         # D = 64 (VALU kernel)
    ("f32", 8, 2, 128, [17, 1, 250], 0),             # fp32
]


@pytest.mark.parametrize("dtype,hq,hkv,d,lengths,partition", EDGE)
def test_fused_edge_shapes(dtype, hq, hkv, d, lengths, partition):
    say(f"append edge dtype={dtype} Hq={hq} Hkv={hkv} D={d} lengths={lengths} partition={partition}")
    wl = kvgen.custom_workload(lengths=lengths, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, dtype=dtype,
                               seed=31, variant="hot", poison=True, table_pad=3)
    ref = oracle.run_step(wl)
    two, fused = _both(wl, partition_size=partition)
    _same(two, fused, "edge")
    check_step(fused, wl, ref, label="edge fused")
    for i, L in enumerate(lengths):
        if L == 0:
            assert not to_f64(fused.out_host()[i], dtype).any(), "zero-length sequence must give zeros"


def test_fused_many_layers_writes_only_its_layer():
    say("3-layer pool, layer 2, fused append")
    wl = kvgen.custom_workload(lengths=[100, 37, 260, 16], num_q_heads=32, num_kv_heads=8, head_dim=128,
                               dtype="bf16", seed=9, variant="sharp", poison=True)
    ref = oracle.run_step(wl)
    from paged_kv_cache_num_amd import DecodeStep
    import torch
    step = DecodeStep.from_workload(wl, num_layers=3, layer=2, partition_size=0)
    step.run_fused()
    torch.cuda.synchronize()
    check_step(step, wl, ref, label="layer 2 of 3, fused")
    for other in (0, 1):
        k, v = step.pool_host(layer=other)
        assert k.tobytes() == wl.k_pool.tobytes() and v.tobytes() == wl.v_pool.tobytes(), "wrote outside its layer"


@pytest.mark.parametrize("name", ["C2", "C3"])
def test_fused_graph_replays_match_eager(name):
    import torch
    say(f"{name} sharp: HIP graph of the fused step")
    wl = workload(name, "sharp")
    two, fused = _both(wl, partition_size=0)
    eager = fused.out_host()
    graph = fused.capture(fused=True)
    for i in range(4):
        fused.out.fill_(0)
        junk = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        del junk
        assert fused.out_host().tobytes() == eager.tobytes(), f"replay {i} differs"
    k2, v2 = two.pool_host()
    kf, vf = fused.pool_host()
    assert kf.tobytes() == k2.tobytes() and vf.tobytes() == v2.tobytes(), "pool after the replays differs"


@pytest.mark.parametrize("B", [8, 64])
def test_step_with_prefill_rows_other_block_sizes(B):
    """paged_attention_decode_step at block sizes other than 16: the extra
    waves that store the 2048-token prefill chunk split each slot with the
    block size's shift.  Bitwise the two-call step, and the oracle."""
    say(f"C3 (48 sequences) at B={B}: step with the prefill chunk vs two calls")
    wl = kvgen.make_workload("C3", variant="sharp", poison=True, num_seqs=48, block_size=B)
    assert wl.extra_tables.shape[0] == 1
    ref = oracle.run_step(wl)
    two, fused = _both(wl, partition_size=0)
    _same(two, fused, f"C3/48/B{B}")
    check_step(fused, wl, ref, label=f"C3/48/B{B} step")
