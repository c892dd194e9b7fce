"""Block sizes other than 16 ("PagedAttention, Internals First", "Why 16?": the
block size trades table lookups against the (B - 1)/2 tokens wasted per
sequence).  bf16 pools with head_dim 128 take B in {8, 16, 32, 64, 128}: the
decode kernels walk 16-token tiles, B/16 per block (B >= 16) or one tile over
two blocks (B = 8).  Scatter bit-exact, attention within tolerance of the
oracle, decode append bitwise equal to scatter + attention."""
import numpy as np
import pytest

import kvgen
import oracle
from parity_util import check_step, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu(gpu_available):
    yield


LENGTHS = [1, 7, 8, 9, 15, 16, 17, 31, 32, 33, 127, 128, 129, 255, 1000, 3001, 0]


@pytest.mark.parametrize("B", [8, 32, 64, 128])
@pytest.mark.parametrize("hq", [32, 64])
@pytest.mark.parametrize("mode", ["balanced", "partitions"])
def test_block_size_parity(B, hq, mode):
    import torch
    from paged_kv_cache_num_amd import DecodeStep
    part = 0 if mode == "balanced" else 2 * max(B, 16)
    say(f"B={B} Hq={hq} Hkv=8 D=128 bf16 {mode} (partition {part})")
    wl = kvgen.custom_workload(lengths=LENGTHS, num_q_heads=hq, num_kv_heads=8, head_dim=128, dtype="bf16",
                               block_size=B, seed=B + hq, variant="hot", poison=True, table_pad=2)
    ref = oracle.run_step(wl)
    two = DecodeStep.from_workload(wl, partition_size=part)
    two.run()
    fused = DecodeStep.from_workload(wl, partition_size=part)
    fused.run_fused()
    torch.cuda.synchronize()
    check_step(two, wl, ref, label=f"B{B}/{mode}")
    check_step(fused, wl, ref, label=f"B{B}/{mode} fused")
    assert fused.out_host().tobytes() == two.out_host().tobytes()


@pytest.mark.parametrize("name,B", [("C2", 8), ("C2", 32), ("C2", 128), ("C5", 64)])
def test_block_size_full_configs(name, B):
    from parity_util import run_gpu
    say(f"{name} at B={B}, balanced split")
    wl = kvgen.make_workload(name, variant="needle", poison=True, block_size=B)
    ref = oracle.run_step(wl)
    step = run_gpu(wl, partition_size=0)
    check_step(step, wl, ref, label=f"{name}/B{B}")


def test_block_size_is_bitwise_placement_invariant():
    from parity_util import run_gpu
    say("C2 at B=32: permuted blocks give the same bits")
    wl = kvgen.make_workload("C2", variant="sharp", poison=True, block_size=32, num_seqs=16)
    base = run_gpu(wl, partition_size=0).out_host()
    perm = run_gpu(kvgen.permute_blocks(wl, 3), partition_size=0).out_host()
    assert np.array_equal(base, perm)
