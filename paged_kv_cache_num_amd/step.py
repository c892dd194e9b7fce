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
    """``dtype`` is the type of q, k_new / v_new and the output.  The pool holds
    the same type, or, with ``fp8_pool = (k_codes, v_codes, k_scale, v_scale)``
    (uint8 ``[N][Hkv][B][D]``, float32 ``[N][Hkv]``), E4M3 codes with block
    scales; dtype is then "bf16" and k_pool / v_pool are not used."""

    def __init__(self, *, k_pool: Optional[np.ndarray], v_pool: Optional[np.ndarray], dtype: str,
                 block_tables: np.ndarray, context_lens: np.ndarray, q: np.ndarray,
                 k_new: np.ndarray, v_new: np.ndarray, write_tables: np.ndarray,
                 write_seq: np.ndarray, write_start: np.ndarray, write_count: np.ndarray,
                 num_layers: int = 1, layer: int = 0, partition_size: int = 0,
                 scale: Optional[float] = None, max_context_len: Optional[int] = None,
                 fp8_pool=None, shared_blocks: int = 0, device="cuda"):
        import torch
        self.fp8 = fp8_pool is not None
        if self.fp8 and dtype != "bf16":
            raise ValueError("FP8 pools take bf16 queries and rows")
        N, Hkv, B, D = (fp8_pool[0] if self.fp8 else k_pool).shape
        self.dtype, self.layer, self.partition_size = dtype, int(layer), int(partition_size)
        self.num_seqs, self.num_q_heads = int(q.shape[0]), int(q.shape[1])
        self.scale = float(scale) if scale is not None else 1.0 / math.sqrt(D)
        self.max_context_len = int(max_context_len if max_context_len is not None
                                   else (context_lens.max() if context_lens.size else 0))
        self.pool = KVPool.allocate(num_layers=num_layers, num_blocks=N, block_size=B,
                                    num_kv_heads=Hkv, head_dim=D,
                                    dtype="fp8" if self.fp8 else (torch.float32 if dtype == "f32" else torch.bfloat16),
                                    device=device)
        # every layer but the working one is filled with the same stale contents
        if self.fp8:
            kc, vc, ks, vs = fp8_pool
            parts = [(self.pool.k, to_device(kc, "u8", device)), (self.pool.v, to_device(vc, "u8", device)),
                     (self.pool.k_scale, to_device(ks, "f32", device)),
                     (self.pool.v_scale, to_device(vs, "f32", device))]
        else:
            parts = [(self.pool.k, to_device(k_pool, dtype, device)), (self.pool.v, to_device(v_pool, dtype, device))]
        for dst, src in parts:
            for li in range(num_layers):
                dst[li].copy_(src)
        del parts
        self.block_tables = to_device(np.ascontiguousarray(block_tables, dtype=np.int32), "i32", device)
        self.context_lens = to_device(np.ascontiguousarray(context_lens, dtype=np.int32), "i32", device)
        self.q = to_device(q, dtype, device)
        self.k_new = to_device(k_new, dtype, device)
        self.v_new = to_device(v_new, dtype, device)
        self.slots_host = kv_build_slot_mapping(write_tables, B, N, write_seq, write_start, write_count)
        self.slot_mapping = to_device(self.slots_host, "i64", device)
        self._split_appends(k_new, v_new, context_lens, write_tables, B, N, write_seq, write_start, write_count,
                            dtype, device)
        self.out = torch.empty_like(self.q)
        # shared_blocks > 0: attend() runs paged_attention_decode_shared (the first
        # shared_blocks table entries of every sequence are the same blocks)
        self.shared_blocks = int(shared_blocks)
        if self.shared_blocks and self.partition_size:
            raise ValueError("a shared prefix goes with partition_size 0")
        if self.shared_blocks:
            ws = self.pool.shared_workspace_bytes(self.num_seqs, self.num_q_heads, self.max_context_len,
                                                  int(block_tables.shape[1]), self.shared_blocks)
        else:
            ws = self.pool.workspace_bytes(self.num_seqs, self.num_q_heads, self.max_context_len,
                                           self.partition_size)
        self.workspace = torch.empty(max(ws, 16), dtype=torch.uint8, device=device) if ws else None

    def _split_appends(self, k_new, v_new, context_lens, write_tables, B, N, write_seq, write_start, write_count,
                       dtype, device):
        """Separate the decode appends (one row per sequence at position L_i - 1,
        for paged_attention_decode_append) from every other write (for
        reshape_and_cache).  ``self.can_fuse`` is False when some sequence with
        L_i > 0 has no such single-row write."""
        S = self.num_seqs
        row0 = np.concatenate([[0], np.cumsum(write_count)]).astype(np.int64)
        seq_row = np.full(S, -1, dtype=np.int64)
        other = []
        for k in range(len(write_seq)):
            i = int(write_seq[k])
            if (i < S and int(write_count[k]) == 1 and int(write_start[k]) == int(context_lens[i]) - 1
                    and seq_row[i] < 0):
                seq_row[i] = row0[k]
            else:
                other.append(k)
        self.can_fuse = bool(all(seq_row[i] >= 0 for i in range(S) if int(context_lens[i]) > 0))
        ak = np.zeros((S,) + k_new.shape[1:], dtype=k_new.dtype)
        av = np.zeros_like(ak)
        has = seq_row >= 0
        ak[has] = k_new[seq_row[has]]
        av[has] = v_new[seq_row[has]]
        self.append_k, self.append_v = to_device(ak, dtype, device), to_device(av, dtype, device)
        rows = (np.concatenate([np.arange(row0[k], row0[k + 1]) for k in other]).astype(np.int64)
                if other else np.zeros(0, dtype=np.int64))
        self.num_other_tokens = int(rows.size)
        if rows.size:
            idx = np.asarray(other)
            slots = kv_build_slot_mapping(write_tables, B, N, np.asarray(write_seq)[idx],
                                          np.asarray(write_start)[idx], np.asarray(write_count)[idx])
            self.other_slots = to_device(slots, "i64", device)
            self.other_k = to_device(np.ascontiguousarray(k_new[rows]), dtype, device)
            self.other_v = to_device(np.ascontiguousarray(v_new[rows]), dtype, device)

    @classmethod
    def from_workload(cls, wl, **kw):
        """kw may carry ``fp8_pool`` (see the class docstring): the step then
        runs on that FP8 pool with ``wl``'s tables, queries and rows."""
        kw.setdefault("partition_size", wl.partition_size)
        return cls(k_pool=wl.k_pool, v_pool=wl.v_pool, dtype=wl.dtype, block_tables=wl.block_tables,
                   context_lens=wl.context_lens, q=wl.q, k_new=wl.k_new, v_new=wl.v_new,
                   write_tables=wl.all_tables(), write_seq=wl.write_seq, write_start=wl.write_start,
                   write_count=wl.write_count, **kw)

    def scatter(self, stream=None):
        self.pool.reshape_and_cache(self.layer, self.k_new, self.v_new, self.slot_mapping, stream=stream)

    def attend(self, stream=None):
        if self.shared_blocks:
            self.pool.paged_attention_decode_shared(self.layer, self.out, self.q, self.block_tables,
                                                    self.context_lens, scale=self.scale,
                                                    max_context_len=self.max_context_len,
                                                    shared_blocks=self.shared_blocks, workspace=self.workspace,
                                                    stream=stream)
            return
        self.pool.paged_attention_decode(self.layer, self.out, self.q, self.block_tables, self.context_lens,
                                         scale=self.scale, max_context_len=self.max_context_len,
                                         partition_size=self.partition_size, workspace=self.workspace,
                                         stream=stream)

    def run(self, stream=None):
        self.scatter(stream)
        self.attend(stream)

    def run_fused(self, stream=None):
        """The same step with the decode appends folded into the attention call
        (paged_attention_decode_append), and the other writes (rows of
        sequences outside the batch, such as a prefill chunk) with them
        (paged_attention_decode_step)."""
        if not self.can_fuse:
            raise ValueError("some sequence has no single-row write at position L_i - 1")
        if self.shared_blocks:
            raise ValueError("the shared-prefix call has no decode-append form")
        if self.num_other_tokens:
            # the other rows (a prefill chunk of a sequence outside the batch) in the same call
            self.pool.paged_attention_decode_step(self.layer, self.out, self.q, self.append_k, self.append_v,
                                                  self.block_tables, self.context_lens, self.other_k, self.other_v,
                                                  self.other_slots, scale=self.scale,
                                                  max_context_len=self.max_context_len,
                                                  partition_size=self.partition_size, workspace=self.workspace,
                                                  stream=stream)
            return
        self.pool.paged_attention_decode_append(self.layer, self.out, self.q, self.append_k, self.append_v,
                                                self.block_tables, self.context_lens, scale=self.scale,
                                                max_context_len=self.max_context_len,
                                                partition_size=self.partition_size, workspace=self.workspace,
                                                stream=stream)

    def capture(self, fused: bool = False):
        """Capture one step (scatter, then attention; with ``fused`` the
        run_fused form) in a HIP graph.

        Every launch of the step reads and writes buffers at fixed addresses
        and allocates nothing, so the step can be captured once and replayed;
        ``graph.replay()`` then runs the whole step with one submission.  The
        step is run once on a side stream first, so that first-call set-up in
        the library (its per-device worker count) happens outside the capture.
        """
        import torch
        body = self.run_fused if fused else self.run
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            body()
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            body()
        return graph

    def out_host(self) -> np.ndarray:
        return to_host(self.out, self.dtype)

    def pool_host(self, layer: Optional[int] = None):
        """K and V of one layer in storage form (FP8 pools: the uint8 codes)."""
        li = self.layer if layer is None else layer
        dt = "u8" if self.fp8 else self.dtype
        return to_host(self.pool.k[li], dt), to_host(self.pool.v[li], dt)

    def scales_host(self, layer: Optional[int] = None):
        """FP8 pools: the K and V block scales of one layer, float32 [N][Hkv]."""
        li = self.layer if layer is None else layer
        return to_host(self.pool.k_scale[li], "f32"), to_host(self.pool.v_scale[li], "f32")
