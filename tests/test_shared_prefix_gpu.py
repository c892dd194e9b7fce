"""GPU parity of paged_attention_decode_shared: a batch whose first table
entries are one common prefix (aicassindra.com "GPU paged KV cache", "Prefix
sharing, reference counts, and copy-on-write"; "PagedAttention, Internals
First", "03 Sharing via copy-on-write").  The call must give what plain
paged decode attention gives over the same tables: it is checked against the
fp64 oracle (which reads through the tables and knows nothing of the
sharing) and against paged_attention_decode itself."""
import dataclasses

import numpy as np
import pytest

import kvgen
import oracle
from parity_util import TOL, check_step, max_err, run_gpu, say, to_f64

pytestmark = pytest.mark.gpu

PREFIX = 2048 // 16   # the C4 workload's prompt: 128 blocks of 16 tokens


def c4_like(hq, lengths, variant, seed):
    shape = kvgen.Shape("C4", kvgen.BF16, hq, 8, 128, 16, 1.0)
    return kvgen.make_workload("C4", seed=seed, variant=variant, poison=True, lengths=np.asarray(lengths),
                               shape=shape)


def plain_and_shared(wl, shared_blocks):
    plain = run_gpu(wl, partition_size=0)
    shared = run_gpu(wl, partition_size=0, shared_blocks=shared_blocks)
    return plain, shared


# lengths: one sequence ends exactly at the prefix (nothing after it), others
# 1, 15, 16, 17 and a few hundred tokens past it; batches that leave the last
# column block of sixteen query heads partly empty
LENGTHS = [2048, 2049, 2048 + 15, 2048 + 16, 2048 + 17, 2048 + 300, 2048 + 512]


@pytest.mark.parametrize("hq", [8, 16, 32, 64])
@pytest.mark.parametrize("variant", ["sharp", "hot"])
def test_shared_prefix_parity(hq, variant):
    say(f"shared prefix: Hq={hq} Hkv=8 lengths={LENGTHS} {variant}")
    wl = c4_like(hq, LENGTHS, variant, seed=hq)
    ref = oracle.run_step(wl)
    plain, shared = plain_and_shared(wl, PREFIX)
    check_step(shared, wl, ref, label=f"shared/Hq{hq}/{variant}")
    d = float(np.abs(to_f64(shared.out_host(), "bf16") - to_f64(plain.out_host(), "bf16")).max())
    say(f"  max |shared - plain| = {d:.3e}")
    assert d <= TOL["bf16"]


def test_shared_prefix_needles_on_both_sides():
    """One key per (sequence, KV head) aligned with a query head: a missed
    prefix tile or a missed suffix tile gives an O(1) error."""
    say("shared prefix: needle variant")
    wl = c4_like(32, [2100, 2300, 2560, 2049, 3000], "needle", seed=5)
    ref = oracle.run_step(wl)
    _, shared = plain_and_shared(wl, PREFIX)
    check_step(shared, wl, ref, label="shared/needle")


def test_shared_prefix_full_c4():
    """The 128-sequence prefix-sharing batch: pool bit-exact after the
    scatter, every output within tolerance of the oracle."""
    say("shared prefix: full C4 batch (128 sequences)")
    wl = kvgen.make_workload("C4", variant="sharp", poison=True)
    assert wl.info["shared_prefix_blocks"] == PREFIX
    ref = oracle.run_step(wl)
    shared = run_gpu(wl, partition_size=0, shared_blocks=PREFIX)
    check_step(shared, wl, ref, label="C4 shared")


def test_shared_prefix_shorter_than_the_tables_share():
    """The call may name fewer shared blocks than the tables have in common."""
    say("shared prefix: 37 of the 128 common blocks named")
    wl = c4_like(32, LENGTHS, "sharp", seed=11)
    ref = oracle.run_step(wl)
    shared = run_gpu(wl, partition_size=0, shared_blocks=37)
    check_step(shared, wl, ref, label="shared 37")


def test_small_prefix_on_an_aliased_batch():
    """Any batch whose rows share their first entries: an 8B-shaped batch of
    ragged lengths with the first three entries of every row pointed at row
    0's blocks (row 0's context covers them, so they hold live data)."""
    say("shared prefix: three aliased blocks on a ragged 8B-shaped batch")
    base = kvgen.custom_workload(lengths=[700, 49, 64, 1000, 300, 2000, 65, 48], num_q_heads=32, num_kv_heads=8,
                                 head_dim=128, dtype="bf16", seed=3, variant="sharp", poison=True)
    tables = base.block_tables.copy()
    tables[:, :3] = tables[0, :3]
    wl = dataclasses.replace(base, block_tables=tables)
    ref = oracle.run_step(wl)
    plain, shared = plain_and_shared(wl, 3)
    check_step(shared, wl, ref, label="aliased 3")
    assert max_err(plain.out_host(), ref["out"], "bf16") <= TOL["bf16"]


def test_zero_shared_blocks_is_the_plain_call_bitwise():
    say("shared_blocks = 0: bitwise the plain balanced call")
    wl = c4_like(32, LENGTHS, "hot", seed=2)
    plain, shared = plain_and_shared(wl, 0)
    assert shared.out_host().tobytes() == plain.out_host().tobytes()


def test_shared_prefix_is_bitwise_placement_invariant_and_repeatable():
    say("shared prefix: bitwise the same over repeated calls and another placement of the blocks")
    wl = c4_like(32, LENGTHS, "sharp", seed=9)
    a = run_gpu(wl, partition_size=0, shared_blocks=PREFIX).out_host()
    b = run_gpu(wl, partition_size=0, shared_blocks=PREFIX).out_host()
    c = run_gpu(kvgen.permute_blocks(wl, 4), partition_size=0, shared_blocks=PREFIX).out_host()
    assert a.tobytes() == b.tobytes()
    assert a.tobytes() == c.tobytes()


def test_shared_prefix_graph_replay():
    """The call captured in a HIP graph and replayed several times, with
    eager work between the replays, leaves the eager call's bits each time."""
    import torch
    from paged_kv_cache_num_amd import DecodeStep
    say("shared prefix: graph replays vs eager")
    wl = c4_like(32, LENGTHS, "sharp", seed=13)
    step = DecodeStep.from_workload(wl, partition_size=0, shared_blocks=PREFIX)
    step.run()
    torch.cuda.synchronize()
    want = step.out_host().tobytes()
    g = step.capture()
    for _ in range(4):
        step.out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert step.out_host().tobytes() == want
        step.attend()
        torch.cuda.synchronize()


@pytest.mark.parametrize("B,shared_blocks", [(8, 256), (8, 255), (32, 64), (64, 32), (128, 16)])
def test_shared_prefix_other_block_sizes(B, shared_blocks):
    """Block sizes 8..128: the prefix waves take the prefix's whole 16-token
    tiles (with 8-token blocks an odd last block is read by the per-sequence
    walks); oracle parity and agreement with the plain call."""
    say(f"shared prefix: B={B} shared_blocks={shared_blocks}")
    shape = kvgen.Shape("C4", kvgen.BF16, 32, 8, 128, B, 1.0)
    wl = kvgen.make_workload("C4", seed=B, variant="sharp", poison=True, lengths=np.asarray(LENGTHS), shape=shape)
    assert wl.info["shared_prefix_blocks"] == 2048 // B
    ref = oracle.run_step(wl)
    plain, shared = plain_and_shared(wl, shared_blocks)
    check_step(shared, wl, ref, label=f"shared/B{B}/{shared_blocks}")
    d = float(np.abs(to_f64(shared.out_host(), "bf16") - to_f64(plain.out_host(), "bf16")).max())
    say(f"  max |shared - plain| = {d:.3e}")
    assert d <= TOL["bf16"]


def test_shared_prefix_full_c4_at_block_size_32():
    say("shared prefix: full C4 batch at B = 32")
    wl = kvgen.make_workload("C4", variant="sharp", poison=True, block_size=32)
    assert wl.info["shared_prefix_blocks"] == 64
    ref = oracle.run_step(wl)
    shared = run_gpu(wl, partition_size=0, shared_blocks=64)
    check_step(shared, wl, ref, label="C4 shared B32")


def test_shared_prefix_block_size_8_odd_row_tail():
    """B = 8 with a 256-block prefix and 293-entry rows: 37 entries follow the
    prefix (an odd count), and the last two sequences fill their rows with
    walks that end in the first half of a 16-token tile (L mod 16 = 7 and 8).
    The walks and the next-walk prefetch read no table entry past the row (the
    last row ends the table buffer); results against the oracle and the plain
    call."""
    lengths = [2100, 2049, 2300, 2343, 2344]
    say(f"shared prefix: B=8, odd row tail, lengths={lengths}")
    shape = kvgen.Shape("C4", kvgen.BF16, 32, 8, 128, 8, 1.0)
    wl = kvgen.make_workload("C4", seed=21, variant="sharp", poison=True, lengths=np.asarray(lengths), shape=shape)
    assert wl.info["shared_prefix_blocks"] == 256
    assert wl.max_blocks_per_seq == 293 and (293 - 256) % 2 == 1
    ref = oracle.run_step(wl)
    plain, shared = plain_and_shared(wl, 256)
    check_step(shared, wl, ref, label="shared/B8/odd tail")
    d = float(np.abs(to_f64(shared.out_host(), "bf16") - to_f64(plain.out_host(), "bf16")).max())
    say(f"  max |shared - plain| = {d:.3e}")
    assert d <= TOL["bf16"]
