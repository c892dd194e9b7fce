"""Measurement probes on the GPU: the copy and read probes move exactly their
bytes, and the table-walk probe reads exactly the block-table entries of the
balanced decode's slices (checked against a host walk of the same slices)."""
import numpy as np
import pytest

import kvgen
from parity_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu(gpu_available):
    yield


def _cum(w):
    # the bf16 decode's slice weights: 33 tiles on an even XCD for 32 on an odd one
    return 33 * ((w + 1) // 2) + 32 * (w // 2)


PIECE_COST = 2   # split positions before each (sequence, KV head) walk's tiles (bf16 tiles)


def _host_walk(tables, lens, hkv, max_context, W, grouped):
    """Per-worker folded word: XOR over walked entries of (entry + kv), as
    uint32.  The split list gives each walk of n > 0 tiles n + PIECE_COST
    positions, the first PIECE_COST of which stand for no tile."""
    lens = np.clip(lens, 0, max_context)
    nblk = (lens + 15) // 16
    span = np.where(nblk > 0, nblk + PIECE_COST, 0)
    T = int(hkv * span.sum())
    starts = np.concatenate([[0], np.cumsum(hkv * span)])
    out = np.zeros(W, dtype=np.uint32)
    for w in range(W):
        s = (w % 8) * (W // 8) + w // 8 if grouped else w
        t0, t1 = T * _cum(s) // _cum(W), T * _cum(s + 1) // _cum(W)
        acc = np.uint32(0)
        for t in range(t0, t1):
            seq = int(np.searchsorted(starts, t, side="right") - 1)
            off = t - starts[seq]
            kv, at = divmod(off, int(span[seq]))
            if at >= PIECE_COST:
                acc ^= np.uint32((int(tables[seq, at - PIECE_COST]) + kv) & 0xFFFFFFFF)
        out[w] = acc
    return out


@pytest.mark.parametrize("grouped", [False, True])
@pytest.mark.parametrize("lengths", [[517, 0, 33, 4096, 16, 1], [3000] * 40])
def test_table_walk_probe_reads_the_decode_slices(grouped, lengths):
    import torch
    from paged_kv_cache_num_amd import probe_table_walk
    say(f"table-walk probe lengths={lengths[:6]}.. grouped={grouped}")
    wl = kvgen.custom_workload(lengths=lengths, num_q_heads=32, num_kv_heads=8, head_dim=128,
                               dtype="bf16", seed=3, variant="spec", poison=False)
    tables = torch.from_numpy(np.ascontiguousarray(wl.block_tables, dtype=np.int32)).cuda()
    lens = torch.from_numpy(np.ascontiguousarray(wl.context_lens, dtype=np.int32)).cuda()
    max_ctx = int(wl.context_lens.max())
    sink = torch.zeros(1 << 14, dtype=torch.uint8, device="cuda")
    probe_table_walk(tables, lens, 8, max_ctx, sink, xcd_grouped=grouped)
    torch.cuda.synchronize()
    got = sink.view(torch.int32).cpu().numpy().view(np.uint32)
    W = int(torch.cuda.get_device_properties(0).multi_processor_count) * 4
    want = _host_walk(wl.block_tables, wl.context_lens, 8, max_ctx, W, grouped)
    assert np.array_equal(got[:W], want)
