"""One decode step's device buffers, kept together: pool, tables, lengths,
queries, new K/V, slot mapping, output and split workspace.

The host builds the slot mapping with the library's kv_build_slot_mapping
(aicassindra.com "GPU paged KV cache", "The write path": the scheduler builds
it on the host each step) and uploads it, with the tables and lengths, into
device buffers that stay at fixed addresses; ``run`` then queues the scatter
and the decode attention on one stream.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

from .kvpool import KVPool, kv_build_slot_mapping


def to_device(a: np.ndarray, dtype: str, device="cuda"):
    """Host array in storage form (float32, or bfloat16 bit patterns as uint16) -> device tensor."""
    import torch
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    elif dtype == "f32":
        t = torch.from_numpy(a.astype(np.float32, copy=False))
    else:
        t = torch.from_numpy(a)
    return t.to(device)


def to_host(t, dtype: str) -> np.ndarray:
    """Device tensor -> host array in storage form."""
    import torch
    t = t.detach().cpu().contiguous()
    if dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


class DecodeStep:
    def __init__(self, *, k_pool: np.ndarray, v_pool: np.ndarray, dtype: str,
                 block_tables: np.ndarray, context_lens: np.ndarray, q: np.ndarray,
                 k_new: np.ndarray, v_new: np.ndarray, write_tables: np.ndarray,
                 write_seq: np.ndarray, write_start: np.ndarray, write_count: np.ndarray,
                 num_layers: int = 1, layer: int = 0, partition_size: int = 0,
                 scale: Optional[float] = None, max_context_len: Optional[int] = None,
                 device="cuda"):
        import torch
        N, Hkv, B, D = k_pool.shape
        self.dtype, self.layer, self.partition_size = dtype, int(layer), int(partition_size)
        self.num_seqs, self.num_q_heads = int(q.shape[0]), int(q.shape[1])
        self.scale = float(scale) if scale is not None else 1.0 / math.sqrt(D)
        self.max_context_len = int(max_context_len if max_context_len is not None
                                   else (context_lens.max() if context_lens.size else 0))
        self.pool = KVPool.allocate(num_layers=num_layers, num_blocks=N, block_size=B,
                                    num_kv_heads=Hkv, head_dim=D,
                                    dtype=torch.float32 if dtype == "f32" else torch.bfloat16,
                                    device=device)
        # every layer but the working one is filled with the same stale contents
        kd, vd = to_device(k_pool, dtype, device), to_device(v_pool, dtype, device)
        for li in range(num_layers):
            self.pool.k[li].copy_(kd)
            self.pool.v[li].copy_(vd)
        del kd, vd
        self.block_tables = to_device(np.ascontiguousarray(block_tables, dtype=np.int32), "i32", device)
        self.context_lens = to_device(np.ascontiguousarray(context_lens, dtype=np.int32), "i32", device)
        self.q = to_device(q, dtype, device)
        self.k_new = to_device(k_new, dtype, device)
        self.v_new = to_device(v_new, dtype, device)
        self.slots_host = kv_build_slot_mapping(write_tables, B, N, write_seq, write_start, write_count)
        self.slot_mapping = to_device(self.slots_host, "i64", device)
        self.out = torch.empty_like(self.q)
        ws = self.pool.workspace_bytes(self.num_seqs, self.num_q_heads, self.max_context_len,
                                       self.partition_size)
        self.workspace = torch.empty(max(ws, 16), dtype=torch.uint8, device=device) if ws else None

    @classmethod
    def from_workload(cls, wl, **kw):
        kw.setdefault("partition_size", wl.partition_size)
        return cls(k_pool=wl.k_pool, v_pool=wl.v_pool, dtype=wl.dtype, block_tables=wl.block_tables,
                   context_lens=wl.context_lens, q=wl.q, k_new=wl.k_new, v_new=wl.v_new,
                   write_tables=wl.all_tables(), write_seq=wl.write_seq, write_start=wl.write_start,
                   write_count=wl.write_count, **kw)

    def scatter(self, stream=None):
        self.pool.reshape_and_cache(self.layer, self.k_new, self.v_new, self.slot_mapping, stream=stream)

    def attend(self, stream=None):
        self.pool.paged_attention_decode(self.layer, self.out, self.q, self.block_tables, self.context_lens,
                                         scale=self.scale, max_context_len=self.max_context_len,
                                         partition_size=self.partition_size, workspace=self.workspace,
                                         stream=stream)

    def run(self, stream=None):
        self.scatter(stream)
        self.attend(stream)

    def capture(self):
        """Capture one step (scatter, then attention) in a HIP graph.

        Every launch of the step reads and writes buffers at fixed addresses
        and allocates nothing, so the step can be captured once and replayed;
        ``graph.replay()`` then runs the whole step with one submission.  The
        step is run once on a side stream first, so that first-call set-up in
        the library (its per-device worker count) happens outside the capture.
        """
        import torch
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self.run()
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            self.run()
        return graph

    def out_host(self) -> np.ndarray:
        return to_host(self.out, self.dtype)

    def pool_host(self, layer: Optional[int] = None):
        li = self.layer if layer is None else layer
        return to_host(self.pool.k[li], self.dtype), to_host(self.pool.v[li], self.dtype)
