"""Python binding of libkvpool.so: argument marshalling only.

Every step of the hot path runs in the HIP library; this module turns torch
tensors (device memory) and numpy arrays (host vectors) into the plain
pointers and sizes the C ABI takes, and turns error codes into exceptions.
There is no fallback: if the library is missing, importing this module fails.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvpool.so")

KV_OK = 0
KV_ERR_INVALID_ARGUMENT = -1
KV_ERR_UNSUPPORTED = -2
KV_ERR_WORKSPACE_TOO_SMALL = -3
KV_ERR_HIP = -4
KV_ERR_OUT_OF_RANGE = -5

KV_NOALLOC_SCRATCH_BYTES = 64 << 20   # the static workspace of paged_attention_decode_noalloc

KV_F32 = 0
KV_BF16 = 1
KV_FP8_E4M3 = 2

# every entry point include/kvpool.h declares
EXPORTED = (
    "kv_pool_bytes", "kv_pool_scale_bytes", "kv_pool_create", "kv_pool_create_fp8", "kv_pool_destroy",
    "kv_build_slot_mapping",
    "reshape_and_cache", "paged_attention_workspace_bytes", "paged_attention_decode",
    "paged_attention_decode_append", "paged_attention_decode_shared", "paged_attention_shared_workspace_bytes",
    "paged_attention_decode_noalloc", "paged_attention_decode_step",
    "kv_copy_blocks", "kv_swap_bytes", "kv_swap_out", "kv_swap_in",
    "kv_status_string", "kv_last_error_message", "kv_probe_copy", "kv_probe_read", "kv_probe_table_walk",
    "kv_probe_e4m3_to_bf16", "kv_probe_f32_to_e4m3",
)


class KVError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: {_status_name(status)}: {detail}")
        self.status = status


class kv_pool_desc(ctypes.Structure):
    _fields_ = [("num_layers", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run `python -m paged_kv_cache_num_amd.build` "
                          "(the HIP library is required; there is no CPU fallback)")
    # torch ships its own HIP runtime under the same soname (libamdhip64.so.7).
    # Loading torch first makes this library bind to that one copy; loading it
    # first would put two HIP runtimes in the process, and the second one to
    # initialise sees no device.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    i32, i64, u64, f32, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_float, ctypes.c_void_p
    P = ctypes.POINTER
    lib.kv_status_string.restype = ctypes.c_char_p
    lib.kv_status_string.argtypes = [ctypes.c_int]
    lib.kv_last_error_message.restype = ctypes.c_char_p
    lib.kv_last_error_message.argtypes = []
    lib.kv_pool_bytes.restype = ctypes.c_int
    lib.kv_pool_bytes.argtypes = [P(kv_pool_desc), P(u64)]
    lib.kv_pool_create.restype = ctypes.c_int
    lib.kv_pool_create.argtypes = [P(kv_pool_desc), vp, vp, P(vp)]
    lib.kv_pool_scale_bytes.restype = ctypes.c_int
    lib.kv_pool_scale_bytes.argtypes = [P(kv_pool_desc), P(u64)]
    lib.kv_pool_create_fp8.restype = ctypes.c_int
    lib.kv_pool_create_fp8.argtypes = [P(kv_pool_desc), vp, vp, vp, vp, P(vp)]
    lib.kv_pool_destroy.restype = ctypes.c_int
    lib.kv_pool_destroy.argtypes = [vp]
    lib.kv_build_slot_mapping.restype = ctypes.c_int
    lib.kv_build_slot_mapping.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, i32, vp, i64, P(i64)]
    lib.reshape_and_cache.restype = ctypes.c_int
    lib.reshape_and_cache.argtypes = [vp, i32, vp, vp, vp, i64, vp]
    lib.paged_attention_workspace_bytes.restype = ctypes.c_int
    lib.paged_attention_workspace_bytes.argtypes = [vp, i32, i32, i32, i32, P(u64)]
    lib.paged_attention_decode.restype = ctypes.c_int
    lib.paged_attention_decode.argtypes = [vp, i32, vp, vp, vp, i32, vp, i32, i32, f32, i32, i32, vp, u64, vp]
    lib.kv_copy_blocks.restype = ctypes.c_int
    lib.kv_copy_blocks.argtypes = [vp, vp, i32, vp]
    lib.kv_swap_bytes.restype = ctypes.c_int
    lib.kv_swap_bytes.argtypes = [vp, i32, P(u64)]
    lib.kv_swap_out.restype = ctypes.c_int
    lib.kv_swap_out.argtypes = [vp, vp, i32, vp, u64, vp]
    lib.kv_swap_in.restype = ctypes.c_int
    lib.kv_swap_in.argtypes = [vp, vp, i32, vp, u64, vp]
    lib.paged_attention_decode_shared.restype = ctypes.c_int
    lib.paged_attention_decode_shared.argtypes = [vp, i32, vp, vp, vp, i32, vp, i32, i32, f32, i32, i32, vp, u64, vp]
    lib.paged_attention_shared_workspace_bytes.restype = ctypes.c_int
    lib.paged_attention_shared_workspace_bytes.argtypes = [vp, i32, i32, i32, i32, i32, P(u64)]
    lib.paged_attention_decode_append.restype = ctypes.c_int
    lib.paged_attention_decode_append.argtypes = [vp, i32, vp, vp, vp, vp, vp, i32, vp, i32, i32, f32, i32, i32,
                                                  vp, u64, vp]
    lib.paged_attention_decode_step.restype = ctypes.c_int
    lib.paged_attention_decode_step.argtypes = [vp, i32, vp, vp, vp, vp, vp, i32, vp, i32, i32, f32, i32, i32,
                                                vp, vp, vp, i64, vp, u64, vp]
    lib.paged_attention_decode_noalloc.restype = ctypes.c_int
    lib.paged_attention_decode_noalloc.argtypes = [vp, i32, vp, vp, vp, i32, vp, i32, i32, f32, i32, i32, vp]
    lib.kv_probe_copy.restype = ctypes.c_int
    lib.kv_probe_copy.argtypes = [vp, vp, u64, vp]
    lib.kv_probe_read.restype = ctypes.c_int
    lib.kv_probe_read.argtypes = [vp, u64, vp, vp]
    lib.kv_probe_table_walk.restype = ctypes.c_int
    lib.kv_probe_table_walk.argtypes = [vp, i32, vp, i32, i32, i32, i32, vp, u64, vp]
    lib.kv_probe_e4m3_to_bf16.restype = ctypes.c_int
    lib.kv_probe_e4m3_to_bf16.argtypes = [vp, vp, i64, vp]
    lib.kv_probe_f32_to_e4m3.restype = ctypes.c_int
    lib.kv_probe_f32_to_e4m3.argtypes = [vp, vp, i64, vp]
    return lib


lib = _load()


def _status_name(status: int) -> str:
    return lib.kv_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != KV_OK:
        raise KVError(status, where, lib.kv_last_error_message().decode())


def dtype_code(dtype) -> int:
    """'f32' / 'bf16' / 'fp8' / torch.float32 / torch.bfloat16 -> kv_dtype."""
    s = str(dtype)
    if s in ("f32", "torch.float32", "float32"):
        return KV_F32
    if s in ("bf16", "torch.bfloat16", "bfloat16"):
        return KV_BF16
    if s in ("fp8", "e4m3", "fp8_e4m3"):
        return KV_FP8_E4M3
    raise ValueError(f"unsupported dtype {dtype}")


def make_desc(num_layers: int, num_blocks: int, block_size: int, num_kv_heads: int,
              head_dim: int, dtype) -> kv_pool_desc:
    return kv_pool_desc(int(num_layers), int(num_blocks), int(block_size), int(num_kv_heads),
                        int(head_dim), dtype_code(dtype))


def kv_pool_bytes(desc: kv_pool_desc) -> int:
    out = ctypes.c_uint64(0)
    _check(lib.kv_pool_bytes(ctypes.byref(desc), ctypes.byref(out)), "kv_pool_bytes")
    return int(out.value)


def kv_pool_scale_bytes(desc: kv_pool_desc) -> int:
    out = ctypes.c_uint64(0)
    _check(lib.kv_pool_scale_bytes(ctypes.byref(desc), ctypes.byref(out)), "kv_pool_scale_bytes")
    return int(out.value)


def kv_build_slot_mapping(block_tables: np.ndarray, block_size: int, num_blocks: int,
                          write_seq: np.ndarray, write_start: np.ndarray,
                          write_count: np.ndarray) -> np.ndarray:
    """Host step: int64 slot per written token (see include/kvpool.h)."""
    t = np.ascontiguousarray(block_tables, dtype=np.int32)
    ws = np.ascontiguousarray(write_seq, dtype=np.int32)
    wst = np.ascontiguousarray(write_start, dtype=np.int32)
    wc = np.ascontiguousarray(write_count, dtype=np.int32)
    cap = int(wc.clip(min=0).sum()) if wc.size else 0
    out = np.empty(max(cap, 1), dtype=np.int64)
    n = ctypes.c_int64(0)
    _check(lib.kv_build_slot_mapping(t.ctypes.data, int(t.shape[0]), int(t.shape[1]), int(block_size),
                                     int(num_blocks), ws.ctypes.data, wst.ctypes.data, wc.ctypes.data,
                                     int(ws.shape[0]), out.ctypes.data, cap, ctypes.byref(n)),
           "kv_build_slot_mapping")
    return out[:n.value].copy()


def _stream_handle(stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def _dev_ptr(t, name: str, dtype=None) -> int:
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return int(t.data_ptr())


class KVPool:
    """A paged K/V pool: caller-owned device tensors wrapped by the C handle.

    ``k`` and ``v`` are device tensors of ``kv_pool_bytes(desc)`` bytes each,
    viewed as ``[num_layers][num_blocks][num_kv_heads][block_size][head_dim]``:
    float32 or bfloat16 values, or, for an FP8 pool, uint8 E4M3 codes.  An FP8
    pool also takes ``k_scale`` / ``v_scale``, float32
    ``[num_layers][num_blocks][num_kv_heads]``; its q, k_new / v_new and
    outputs are bfloat16 (``torch_dtype``).
    """

    def __init__(self, k, v, *, num_layers: int, num_blocks: int, block_size: int,
                 num_kv_heads: int, head_dim: int, k_scale=None, v_scale=None):
        import torch
        self.fp8 = k.dtype == torch.uint8
        self.desc = make_desc(num_layers, num_blocks, block_size, num_kv_heads, head_dim,
                              "fp8" if self.fp8 else k.dtype)
        need = kv_pool_bytes(self.desc)
        for name, t in (("k", k), ("v", v)):
            if t.dtype != k.dtype or t.numel() * t.element_size() != need:
                raise ValueError(f"{name} pool must hold {need} bytes of {k.dtype}")
        self.k, self.v = k, v
        self.k_scale, self.v_scale = k_scale, v_scale
        self.torch_dtype = torch.bfloat16 if self.fp8 else k.dtype
        self._h = ctypes.c_void_p(0)
        if self.fp8:
            sneed = kv_pool_scale_bytes(self.desc)
            for name, t in (("k_scale", k_scale), ("v_scale", v_scale)):
                if t is None or t.dtype != torch.float32 or t.numel() * 4 != sneed:
                    raise ValueError(f"{name} must be a float32 tensor of {sneed} bytes")
            _check(lib.kv_pool_create_fp8(ctypes.byref(self.desc), _dev_ptr(k, "k"), _dev_ptr(v, "v"),
                                          _dev_ptr(k_scale, "k_scale"), _dev_ptr(v_scale, "v_scale"),
                                          ctypes.byref(self._h)), "kv_pool_create_fp8")
        else:
            _check(lib.kv_pool_create(ctypes.byref(self.desc), _dev_ptr(k, "k"), _dev_ptr(v, "v"),
                                      ctypes.byref(self._h)), "kv_pool_create")
        self.num_layers, self.num_blocks, self.block_size = num_layers, num_blocks, block_size
        self.num_kv_heads, self.head_dim = num_kv_heads, head_dim

    @classmethod
    def allocate(cls, *, num_layers: int, num_blocks: int, block_size: int, num_kv_heads: int,
                 head_dim: int, dtype, device="cuda"):
        """dtype: torch.float32, torch.bfloat16, or "fp8" (uint8 codes plus float32 scales)."""
        import torch
        shape = (num_layers, num_blocks, num_kv_heads, block_size, head_dim)
        if str(dtype) in ("fp8", "e4m3", "fp8_e4m3"):
            k = torch.empty(shape, dtype=torch.uint8, device=device)
            v = torch.empty(shape, dtype=torch.uint8, device=device)
            ks = torch.ones(shape[:3], dtype=torch.float32, device=device)
            vs = torch.ones(shape[:3], dtype=torch.float32, device=device)
            return cls(k, v, num_layers=num_layers, num_blocks=num_blocks, block_size=block_size,
                       num_kv_heads=num_kv_heads, head_dim=head_dim, k_scale=ks, v_scale=vs)
        k = torch.empty(shape, dtype=dtype, device=device)
        v = torch.empty(shape, dtype=dtype, device=device)
        return cls(k, v, num_layers=num_layers, num_blocks=num_blocks, block_size=block_size,
                   num_kv_heads=num_kv_heads, head_dim=head_dim)

    @property
    def handle(self) -> int:
        return int(self._h.value or 0)

    def close(self):
        if self._h.value:
            lib.kv_pool_destroy(self._h)
            self._h = ctypes.c_void_p(0)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- GPU steps ------------------------------------------------------
    def reshape_and_cache(self, layer: int, k_new, v_new, slot_mapping, stream=None) -> None:
        import torch
        T = int(slot_mapping.shape[0])
        row = (T, self.num_kv_heads, self.head_dim)
        if tuple(k_new.shape) != row or tuple(v_new.shape) != row:
            raise ValueError(f"k_new/v_new must be {row}")
        _check(lib.reshape_and_cache(self.handle, int(layer),
                                     _dev_ptr(k_new, "k_new", self.torch_dtype),
                                     _dev_ptr(v_new, "v_new", self.torch_dtype),
                                     _dev_ptr(slot_mapping, "slot_mapping", torch.int64), T,
                                     _stream_handle(stream)), "reshape_and_cache")

    def workspace_bytes(self, num_seqs: int, num_q_heads: int, max_context_len: int,
                        partition_size: int) -> int:
        out = ctypes.c_uint64(0)
        _check(lib.paged_attention_workspace_bytes(self.handle, int(num_seqs), int(num_q_heads),
                                                   int(max_context_len), int(partition_size),
                                                   ctypes.byref(out)), "paged_attention_workspace_bytes")
        return int(out.value)

    def paged_attention_decode(self, layer: int, out, q, block_tables, context_lens, *,
                               scale: float, max_context_len: int, partition_size: int = 0,
                               workspace=None, stream=None) -> None:
        import torch
        S, Hq, D = (int(x) for x in q.shape)
        if tuple(out.shape) != (S, Hq, D) or D != self.head_dim:
            raise ValueError("q/out must be [num_seqs][num_q_heads][head_dim]")
        if block_tables.dim() != 2 or block_tables.shape[0] != S or tuple(context_lens.shape) != (S,):
            raise ValueError("one table row and one length per sequence")
        ws_ptr, ws_bytes = None, 0
        if workspace is not None:
            ws_ptr = _dev_ptr(workspace, "workspace")
            ws_bytes = workspace.numel() * workspace.element_size()
        _check(lib.paged_attention_decode(self.handle, int(layer),
                                          _dev_ptr(out, "out", self.torch_dtype),
                                          _dev_ptr(q, "q", self.torch_dtype),
                                          _dev_ptr(block_tables, "block_tables", torch.int32),
                                          int(block_tables.shape[1]),
                                          _dev_ptr(context_lens, "context_lens", torch.int32),
                                          S, Hq, float(scale), int(max_context_len), int(partition_size),
                                          ws_ptr, int(ws_bytes), _stream_handle(stream)),
               "paged_attention_decode")

    def paged_attention_decode_noalloc(self, layer: int, out, q, block_tables, context_lens, *,
                                       scale: float, max_context_len: int, partition_size: int = 0,
                                       stream=None) -> None:
        """paged_attention_decode with the library's static per-device workspace
        (allocates nothing; calls overlapping on one GPU race)."""
        import torch
        S, Hq, D = (int(x) for x in q.shape)
        if tuple(out.shape) != (S, Hq, D) or D != self.head_dim:
            raise ValueError("q/out must be [num_seqs][num_q_heads][head_dim]")
        if block_tables.dim() != 2 or block_tables.shape[0] != S or tuple(context_lens.shape) != (S,):
            raise ValueError("one table row and one length per sequence")
        _check(lib.paged_attention_decode_noalloc(self.handle, int(layer),
                                                  _dev_ptr(out, "out", self.torch_dtype),
                                                  _dev_ptr(q, "q", self.torch_dtype),
                                                  _dev_ptr(block_tables, "block_tables", torch.int32),
                                                  int(block_tables.shape[1]),
                                                  _dev_ptr(context_lens, "context_lens", torch.int32),
                                                  S, Hq, float(scale), int(max_context_len), int(partition_size),
                                                  _stream_handle(stream)),
               "paged_attention_decode_noalloc")

    def shared_workspace_bytes(self, num_seqs: int, num_q_heads: int, max_context_len: int,
                               max_blocks_per_seq: int, shared_blocks: int) -> int:
        out = ctypes.c_uint64(0)
        _check(lib.paged_attention_shared_workspace_bytes(self.handle, int(num_seqs), int(num_q_heads),
                                                          int(max_context_len), int(max_blocks_per_seq),
                                                          int(shared_blocks), ctypes.byref(out)),
               "paged_attention_shared_workspace_bytes")
        return int(out.value)

    def paged_attention_decode_shared(self, layer: int, out, q, block_tables, context_lens, *,
                                      scale: float, max_context_len: int, shared_blocks: int,
                                      workspace=None, stream=None) -> None:
        """paged_attention_decode for a batch whose first ``shared_blocks``
        table entries are common to every sequence (see the C header)."""
        import torch
        S, Hq, D = (int(x) for x in q.shape)
        if tuple(out.shape) != (S, Hq, D) or D != self.head_dim:
            raise ValueError("q/out must be [num_seqs][num_q_heads][head_dim]")
        if block_tables.dim() != 2 or block_tables.shape[0] != S or tuple(context_lens.shape) != (S,):
            raise ValueError("one table row and one length per sequence")
        ws_ptr, ws_bytes = None, 0
        if workspace is not None:
            ws_ptr = _dev_ptr(workspace, "workspace")
            ws_bytes = workspace.numel() * workspace.element_size()
        _check(lib.paged_attention_decode_shared(self.handle, int(layer),
                                                 _dev_ptr(out, "out", self.torch_dtype),
                                                 _dev_ptr(q, "q", self.torch_dtype),
                                                 _dev_ptr(block_tables, "block_tables", torch.int32),
                                                 int(block_tables.shape[1]),
                                                 _dev_ptr(context_lens, "context_lens", torch.int32),
                                                 S, Hq, float(scale), int(max_context_len), int(shared_blocks),
                                                 ws_ptr, int(ws_bytes), _stream_handle(stream)),
               "paged_attention_decode_shared")

    def copy_blocks(self, block_pairs, stream=None) -> None:
        """Copy-on-write device copy: block src -> block dst in every layer of K and V.

        ``block_pairs``: int32 device tensor [num_pairs][2] of (src, dst)."""
        import torch
        if block_pairs.dim() != 2 or block_pairs.shape[1] != 2:
            raise ValueError("block_pairs must be [num_pairs][2]")
        n = int(block_pairs.shape[0])
        ptr = _dev_ptr(block_pairs, "block_pairs", torch.int32) if n else None
        _check(lib.kv_copy_blocks(self.handle, ptr, n, _stream_handle(stream)), "kv_copy_blocks")

    def swap_bytes(self, num_blocks: int) -> int:
        """Host bytes that swapping out ``num_blocks`` blocks takes."""
        out = ctypes.c_uint64(0)
        _check(lib.kv_swap_bytes(self.handle, int(num_blocks), ctypes.byref(out)), "kv_swap_bytes")
        return int(out.value)

    def _swap(self, fn, name, blocks, host, stream):
        import torch
        if blocks.dim() != 1:
            raise ValueError("blocks must be a 1-D int32 device tensor")
        if not isinstance(host, torch.Tensor) or host.is_cuda or not host.is_contiguous():
            raise TypeError("host buffer must be a contiguous host tensor (pinned: pin_memory=True)")
        n = int(blocks.shape[0])
        bptr = _dev_ptr(blocks, "blocks", torch.int32) if n else None
        _check(fn(self.handle, bptr, n, host.data_ptr() if host.numel() else None,
                  host.numel() * host.element_size(), _stream_handle(stream)), name)

    def swap_out(self, blocks, host, stream=None) -> None:
        """Copy the listed blocks (every layer, FP8 scales too) into pinned host memory."""
        self._swap(lib.kv_swap_out, "kv_swap_out", blocks, host, stream)

    def swap_in(self, blocks, host, stream=None) -> None:
        """Copy host records back into the listed blocks (every layer)."""
        self._swap(lib.kv_swap_in, "kv_swap_in", blocks, host, stream)

    def paged_attention_decode_append(self, layer: int, out, q, k_new, v_new, block_tables, context_lens, *,
                                      scale: float, max_context_len: int, partition_size: int = 0,
                                      workspace=None, stream=None) -> None:
        """Append each sequence's new K/V row at position L_i - 1 and attend, in one call."""
        import torch
        S, Hq, D = (int(x) for x in q.shape)
        if tuple(out.shape) != (S, Hq, D) or D != self.head_dim:
            raise ValueError("q/out must be [num_seqs][num_q_heads][head_dim]")
        if tuple(k_new.shape) != (S, self.num_kv_heads, D) or tuple(v_new.shape) != (S, self.num_kv_heads, D):
            raise ValueError("k_new/v_new must be [num_seqs][num_kv_heads][head_dim]")
        if block_tables.dim() != 2 or block_tables.shape[0] != S or tuple(context_lens.shape) != (S,):
            raise ValueError("one table row and one length per sequence")
        ws_ptr, ws_bytes = None, 0
        if workspace is not None:
            ws_ptr = _dev_ptr(workspace, "workspace")
            ws_bytes = workspace.numel() * workspace.element_size()
        _check(lib.paged_attention_decode_append(self.handle, int(layer),
                                                 _dev_ptr(out, "out", self.torch_dtype),
                                                 _dev_ptr(q, "q", self.torch_dtype),
                                                 _dev_ptr(k_new, "k_new", self.torch_dtype),
                                                 _dev_ptr(v_new, "v_new", self.torch_dtype),
                                                 _dev_ptr(block_tables, "block_tables", torch.int32),
                                                 int(block_tables.shape[1]),
                                                 _dev_ptr(context_lens, "context_lens", torch.int32),
                                                 S, Hq, float(scale), int(max_context_len), int(partition_size),
                                                 ws_ptr, int(ws_bytes), _stream_handle(stream)),
               "paged_attention_decode_append")

    def paged_attention_decode_step(self, layer: int, out, q, k_new, v_new, block_tables, context_lens,
                                    k_rows, v_rows, row_slots, *, scale: float, max_context_len: int,
                                    partition_size: int = 0, workspace=None, stream=None) -> None:
        """Store other rows (reshape_and_cache of k_rows / v_rows to row_slots),
        append each sequence's new row at position L_i - 1 and attend, in one
        call.  The other rows' slots must lie in blocks the attention does not
        read (a prefill chunk of a sequence outside the batch)."""
        import torch
        S, Hq, D = (int(x) for x in q.shape)
        R = int(row_slots.shape[0])
        if tuple(out.shape) != (S, Hq, D) or D != self.head_dim:
            raise ValueError("q/out must be [num_seqs][num_q_heads][head_dim]")
        if tuple(k_new.shape) != (S, self.num_kv_heads, D) or tuple(v_new.shape) != (S, self.num_kv_heads, D):
            raise ValueError("k_new/v_new must be [num_seqs][num_kv_heads][head_dim]")
        if tuple(k_rows.shape) != (R, self.num_kv_heads, D) or tuple(v_rows.shape) != (R, self.num_kv_heads, D):
            raise ValueError("k_rows/v_rows must be [num_rows][num_kv_heads][head_dim]")
        if block_tables.dim() != 2 or block_tables.shape[0] != S or tuple(context_lens.shape) != (S,):
            raise ValueError("one table row and one length per sequence")
        ws_ptr, ws_bytes = None, 0
        if workspace is not None:
            ws_ptr = _dev_ptr(workspace, "workspace")
            ws_bytes = workspace.numel() * workspace.element_size()
        _check(lib.paged_attention_decode_step(self.handle, int(layer),
                                               _dev_ptr(out, "out", self.torch_dtype),
                                               _dev_ptr(q, "q", self.torch_dtype),
                                               _dev_ptr(k_new, "k_new", self.torch_dtype),
                                               _dev_ptr(v_new, "v_new", self.torch_dtype),
                                               _dev_ptr(block_tables, "block_tables", torch.int32),
                                               int(block_tables.shape[1]),
                                               _dev_ptr(context_lens, "context_lens", torch.int32),
                                               S, Hq, float(scale), int(max_context_len), int(partition_size),
                                               _dev_ptr(k_rows, "k_rows", self.torch_dtype),
                                               _dev_ptr(v_rows, "v_rows", self.torch_dtype),
                                               _dev_ptr(row_slots, "row_slots", torch.int64), R,
                                               ws_ptr, int(ws_bytes), _stream_handle(stream)),
               "paged_attention_decode_step")


def probe_copy(dst, src, stream=None) -> None:
    """Measurement probe: plain device copy of src into dst (same byte size)."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("copy probe needs equal sizes")
    _check(lib.kv_probe_copy(_dev_ptr(dst, "dst"), _dev_ptr(src, "src"), nbytes, _stream_handle(stream)),
           "kv_probe_copy")


def probe_read(src, sink, stream=None) -> None:
    """Measurement probe: read all of src (16-byte loads); sink takes >= 64 KiB of words."""
    if sink.numel() * sink.element_size() < 65536:
        raise ValueError("sink must hold at least 64 KiB")
    _check(lib.kv_probe_read(_dev_ptr(src, "src"), src.numel() * src.element_size(), _dev_ptr(sink, "sink"),
                             _stream_handle(stream)), "kv_probe_read")


def probe_table_walk(block_tables, context_lens, num_kv_heads: int, max_context_len: int, sink, *,
                     xcd_grouped: bool = False, stream=None) -> None:
    """Measurement probe: the balanced decode's block-table walk without the K/V loads."""
    import torch
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32 or block_tables.dim() != 2:
        raise TypeError("block_tables [S][MB] and context_lens [S] must be int32 device tensors")
    _check(lib.kv_probe_table_walk(_dev_ptr(block_tables, "block_tables"), block_tables.shape[1],
                                   _dev_ptr(context_lens, "context_lens"), block_tables.shape[0],
                                   int(num_kv_heads), int(max_context_len), 1 if xcd_grouped else 0,
                                   _dev_ptr(sink, "sink"), sink.numel() * sink.element_size(),
                                   _stream_handle(stream)), "kv_probe_table_walk")


def probe_e4m3_to_bf16(codes, out, stream=None) -> None:
    """Test hook: widen uint8 E4M3 codes to bfloat16 (out: int16/bfloat16 tensor, same length)."""
    import torch
    if codes.dtype != torch.uint8 or out.numel() != codes.numel() or out.element_size() != 2:
        raise TypeError("codes: uint8; out: 2-byte elements, same count")
    _check(lib.kv_probe_e4m3_to_bf16(_dev_ptr(codes, "codes"), _dev_ptr(out, "out"), codes.numel(),
                                     _stream_handle(stream)), "kv_probe_e4m3_to_bf16")


def probe_f32_to_e4m3(x, out, stream=None) -> None:
    """Test hook: fp32 values to E4M3 codes as the FP8 write path rounds them."""
    import torch
    if x.dtype != torch.float32 or out.dtype != torch.uint8 or out.numel() != x.numel():
        raise TypeError("x: float32; out: uint8, same count")
    _check(lib.kv_probe_f32_to_e4m3(_dev_ptr(x, "x"), _dev_ptr(out, "out"), x.numel(), _stream_handle(stream)),
           "kv_probe_f32_to_e4m3")
