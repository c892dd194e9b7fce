"""paged_attention_decode_noalloc: the decode call with the library's static
per-device workspace instead of a caller's buffer.  Called through the C ABI
(the binding only marshals), it must give bitwise the output of
paged_attention_decode on the same inputs (same kernels), and stay within
the oracle's tolerance, on two calls in a row whose second is smaller (the
array keeps the first call's contents)."""
import numpy as np
import pytest

import kvgen
import oracle
from parity_util import TOL, max_err, say

pytestmark = pytest.mark.gpu


def _noalloc_vs_decode(wl, part, fp8_state=None, check_oracle=True):
    import torch
    from paged_kv_cache_num_amd import DecodeStep
    step = DecodeStep.from_workload(wl, partition_size=part, fp8_pool=fp8_state)
    step.run()                                   # scatter, then paged_attention_decode with a workspace
    torch.cuda.synchronize()
    want = step.out_host()
    step.out.fill_(float("nan"))
    step.pool.paged_attention_decode_noalloc(step.layer, step.out, step.q, step.block_tables, step.context_lens,
                                             scale=step.scale, max_context_len=step.max_context_len,
                                             partition_size=part)
    torch.cuda.synchronize()
    got = step.out_host()
    assert got.tobytes() == want.tobytes(), "noalloc output differs from paged_attention_decode"
    if check_oracle:
        if fp8_state is None:
            ref = oracle.run_step(wl)["out"]
        else:
            import oracle.fp8 as ofp8
            kc, vc, ks, vs = ofp8.scatter(*fp8_state, wl.k_new, wl.v_new, step.slots_host, wl.block_size)
            ref = ofp8.paged_attention(wl.q, kc, vc, ks, vs, wl.block_tables, wl.context_lens, step.scale)
        err = max_err(got, ref, wl.dtype)
        say(f"  max |noalloc - oracle| = {err:.3e}")
        assert err <= TOL[wl.dtype]
    del step
    torch.cuda.synchronize()


@pytest.mark.parametrize("part", [0, 512])
def test_noalloc_two_calls_second_smaller(part):
    big = kvgen.make_workload("C2", variant="sharp", poison=True, num_seqs=24)
    small = kvgen.make_workload("C2", seed=7, variant="hot", poison=True, num_seqs=5)
    for wl in (big, small):
        say(f"noalloc: C2-shaped, {wl.num_seqs} sequences, partition {part}")
        _noalloc_vs_decode(wl, part)


def test_noalloc_fp8_group_8_then_smaller():
    """FP8 pool with eight query heads per KV head: the largest balanced workspace."""
    shape = kvgen.Shape("C3", kvgen.BF16, 64, 8, 128, 16, 1.0)
    for S, seed in ((40, 3), (9, 4)):
        wl = kvgen.make_workload("C3", seed=seed, variant="sharp", poison=True, num_seqs=S, shape=shape)
        say(f"noalloc: FP8 pool, G=8, {S} sequences")
        _noalloc_vs_decode(wl, 0, fp8_state=kvgen.fp8_pool_state(wl, seed=seed))


def test_noalloc_long_context_partitions_then_small():
    """The long-context batch with 512-token partitions (about 34 MB of
    workspace), then a small batch: bitwise the workspace call each time."""
    say("noalloc: long-context batch, 512-token partitions")
    _noalloc_vs_decode(kvgen.make_workload("C5", variant="sharp", poison=True), 512, check_oracle=False)
    say("noalloc: then 3 short sequences")
    _noalloc_vs_decode(kvgen.custom_workload(lengths=[1, 17, 300], num_q_heads=32, num_kv_heads=8, head_dim=128,
                                             dtype="bf16", seed=5), 512)
