"""CPU oracle for the paged KV-cache hot path (fp64), Python side.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import this package; the product library
never does.  The arithmetic lives in ``oracle.c`` (plain C, fp64, built with
gcc); this module only marshals numpy arrays into it.

Functions follow the pages' notation: a slot is ``block_index * B + offset``
(aicassindra.com "GPU paged KV cache", "The write path: slot mapping and
scatter"); token t of a sequence lives in logical block ``t // B`` at offset
``t % B`` ("PagedAttention, Internals First", "02 Block tables").

Parity status: every function here is pinned by the ``-m "not gpu"`` tests
(library cross-check, closed forms, invariances, the pages' worked numbers).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")

_lib = None

_DTYPE_CODE = {"f32": 0, "bf16": 1}

_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_f64p = ctypes.POINTER(ctypes.c_double)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    src = os.path.join(HERE, "oracle.c")
    if not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(src):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(LIB_PATH)
    lib.oracle_slot_mapping.restype = ctypes.c_int64
    lib.oracle_slot_mapping.argtypes = [_i32p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int64, _i32p, _i32p, _i32p, ctypes.c_int32,
                                        _i64p, ctypes.c_int64]
    lib.oracle_scatter.restype = ctypes.c_int
    lib.oracle_scatter.argtypes = [_u8p, _u8p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                   ctypes.c_int32, ctypes.c_int32, _u8p, _u8p, _i64p, ctypes.c_int64]
    lib.oracle_paged_attention.restype = ctypes.c_int
    lib.oracle_paged_attention.argtypes = [_f64p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                                           ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                           _i32p, ctypes.c_int32, _i32p, ctypes.c_int32,
                                           ctypes.c_double, ctypes.c_int32]
    _lib = lib
    return lib


def _ptr(a: np.ndarray, typ):
    return a.ctypes.data_as(typ)


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def slot_mapping(tables: np.ndarray, block_size: int, num_blocks: int,
                 write_seq: np.ndarray, write_start: np.ndarray,
                 write_count: np.ndarray) -> np.ndarray:
    """Linear destination of every written token: table[row][p // B] * B + p % B."""
    lib = _load()
    tables = np.ascontiguousarray(tables, dtype=np.int32)
    ws = np.ascontiguousarray(write_seq, dtype=np.int32)
    wst = np.ascontiguousarray(write_start, dtype=np.int32)
    wc = np.ascontiguousarray(write_count, dtype=np.int32)
    cap = int(wc.sum()) if wc.size else 0
    out = np.empty(max(cap, 1), dtype=np.int64)
    n = lib.oracle_slot_mapping(_ptr(tables, _i32p), int(tables.shape[0]), int(tables.shape[1]),
                                int(block_size), int(num_blocks), _ptr(ws, _i32p), _ptr(wst, _i32p),
                                _ptr(wc, _i32p), int(ws.shape[0]), _ptr(out, _i64p), cap)
    if n < 0:
        raise ValueError("write request outside its block table, or table entry outside the pool")
    return out[:n].copy()


def scatter(k_pool: np.ndarray, v_pool: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
            slots: np.ndarray):
    """Return copies of the pools with each token's K/V rows copied to its slot."""
    lib = _load()
    kp = np.ascontiguousarray(k_pool).copy()
    vp = np.ascontiguousarray(v_pool).copy()
    N, H, B, D = kp.shape
    kn = np.ascontiguousarray(k_new)
    vn = np.ascontiguousarray(v_new)
    sl = np.ascontiguousarray(slots, dtype=np.int64)
    if kn.dtype != kp.dtype or vn.dtype != vp.dtype or kn.shape != (sl.shape[0], H, D):
        raise ValueError("k_new/v_new must be [num_tokens][num_kv_heads][head_dim] in the pool dtype")
    rc = lib.oracle_scatter(kp.view(np.uint8).ctypes.data_as(_u8p), vp.view(np.uint8).ctypes.data_as(_u8p),
                            N, H, B, D, kp.dtype.itemsize,
                            kn.view(np.uint8).ctypes.data_as(_u8p), vn.view(np.uint8).ctypes.data_as(_u8p),
                            _ptr(sl, _i64p), int(sl.shape[0]))
    if rc != 0:
        raise ValueError("slot outside the pool")
    return kp, vp


def copy_blocks(k_pool: np.ndarray, v_pool: np.ndarray, pairs):
    """Copy-on-write block copy, plain numpy (aicassindra.com "GPU paged KV
    cache", "Prefix sharing, reference counts, and copy-on-write";
    "PagedAttention, Internals First", "03 Sharing via copy-on-write": the
    shared block's contents are copied into the writer's fresh block).

    Returns copies of the pools in which block ``dst`` holds what block ``src``
    held before the call, for every ``(src, dst)`` pair naming two blocks of the
    pool; pairs naming a block outside it are skipped.  Pools are
    ``[N][Hkv][B][D]`` or carry a leading layers axis (every layer is copied).
    """
    kp, vp = k_pool.copy(), v_pool.copy()
    n = k_pool.shape[-4]
    for src, dst in pairs:
        src, dst = int(src), int(dst)
        if 0 <= src < n and 0 <= dst < n:
            kp[..., dst, :, :, :] = k_pool[..., src, :, :, :]
            vp[..., dst, :, :, :] = v_pool[..., src, :, :, :]
    return kp, vp


def paged_attention(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray, dtype: str,
                    block_tables: np.ndarray, context_lens: np.ndarray, scale: float,
                    threads: Optional[int] = None) -> np.ndarray:
    """fp64 decode attention through block tables; returns [num_seqs][num_q_heads][head_dim]."""
    lib = _load()
    q = np.ascontiguousarray(q)
    kp = np.ascontiguousarray(k_pool)
    vp = np.ascontiguousarray(v_pool)
    N, Hkv, B, D = kp.shape
    S, Hq, Dq = q.shape
    if Dq != D:
        raise ValueError("head_dim mismatch")
    tables = np.ascontiguousarray(block_tables, dtype=np.int32)
    lens = np.ascontiguousarray(context_lens, dtype=np.int32)
    if tables.shape[0] != S or lens.shape[0] != S:
        raise ValueError("one table row and one length per sequence")
    out = np.zeros((S, Hq, D), dtype=np.float64)
    rc = lib.oracle_paged_attention(_ptr(out, _f64p), q.ctypes.data, kp.ctypes.data, vp.ctypes.data,
                                    _DTYPE_CODE[dtype], N, Hkv, B, D, Hq,
                                    _ptr(tables, _i32p), int(tables.shape[1]), _ptr(lens, _i32p), S,
                                    float(scale), int(threads or default_threads()))
    if rc != 0:
        raise ValueError(f"oracle_paged_attention failed ({rc})")
    return out


def run_step(wl, scale: Optional[float] = None, threads: Optional[int] = None,
             seqs: Optional[np.ndarray] = None):
    """One step of the hot path on a ``kvgen.Workload``: slot mapping, scatter, attention.

    ``seqs`` restricts attention to a subset of sequences (sampled outputs).
    Returns ``dict(slots, k_pool, v_pool, out)``.
    """
    if scale is None:
        scale = 1.0 / float(np.sqrt(wl.head_dim))
    slots = slot_mapping(wl.all_tables(), wl.block_size, wl.num_blocks,
                         wl.write_seq, wl.write_start, wl.write_count)
    kp, vp = scatter(wl.k_pool, wl.v_pool, wl.k_new, wl.v_new, slots)
    if seqs is None:
        out = paged_attention(wl.q, kp, vp, wl.dtype, wl.block_tables, wl.context_lens, scale, threads)
    else:
        seqs = np.asarray(seqs)
        out = paged_attention(wl.q[seqs], kp, vp, wl.dtype, wl.block_tables[seqs],
                              wl.context_lens[seqs], scale, threads)
    return dict(slots=slots, k_pool=kp, v_pool=vp, out=out)


def swap_record_bytes(num_layers: int, run_bytes: int, num_kv_heads: int = 0, fp8: bool = False) -> int:
    """Host bytes of one swapped block: its K and V runs of every layer, then
    (FP8) its K and V scales of every layer, padded to a multiple of 16."""
    rec = 2 * num_layers * run_bytes + (2 * num_layers * num_kv_heads * 4 if fp8 else 0)
    return -(-rec // 16) * 16


def swap_out(k_pool: np.ndarray, v_pool: np.ndarray, blocks, k_scale=None, v_scale=None) -> np.ndarray:
    """Swap to host (aicassindra.com "GPU paged KV cache", "Reclaiming memory:
    swap versus recompute"; "PagedAttention, Internals First", "05 Preemption
    and the scheduler contract": the victim's blocks are copied to host memory
    and back on resume), plain numpy.

    Pools are ``[layers][N][Hkv][B][D]`` (any dtype), FP8 scales
    ``[layers][N][Hkv]`` float32.  Returns the host buffer as bytes: one record
    per listed block, in list order, holding for each layer the block's K then
    V bytes, then for each layer its K then V scales, zero-padded to 16 bytes.
    A listed index outside the pool leaves its record zero.
    """
    L, N = k_pool.shape[0], k_pool.shape[1]
    fp8 = k_scale is not None
    H = k_pool.shape[2]
    run = k_pool[0, 0].nbytes
    rec = swap_record_bytes(L, run, H, fp8)
    out = np.zeros((len(blocks), rec), dtype=np.uint8)
    for i, b in enumerate(blocks):
        b = int(b)
        if not 0 <= b < N:
            continue
        parts = []
        for layer in range(L):
            parts += [k_pool[layer, b].tobytes(), v_pool[layer, b].tobytes()]
        if fp8:
            for layer in range(L):
                parts += [np.asarray(k_scale[layer, b], dtype=np.float32).tobytes(),
                          np.asarray(v_scale[layer, b], dtype=np.float32).tobytes()]
        data = b"".join(parts)
        out[i, :len(data)] = np.frombuffer(data, dtype=np.uint8)
    return out.reshape(-1)


def swap_in(k_pool: np.ndarray, v_pool: np.ndarray, blocks, host: np.ndarray, k_scale=None, v_scale=None):
    """Inverse of swap_out: record i of ``host`` goes back to block ``blocks[i]``
    of every layer.  Returns new pools (and new scales for FP8 pools); indices
    outside the pool are skipped."""
    kp, vp = k_pool.copy(), v_pool.copy()
    fp8 = k_scale is not None
    ks = k_scale.copy() if fp8 else None
    vs = v_scale.copy() if fp8 else None
    L, N, H = k_pool.shape[0], k_pool.shape[1], k_pool.shape[2]
    run = k_pool[0, 0].nbytes
    rec = swap_record_bytes(L, run, H, fp8)
    host = np.asarray(host, dtype=np.uint8).reshape(-1, rec)
    tile = k_pool.shape[2:]
    for i, b in enumerate(blocks):
        b = int(b)
        if not 0 <= b < N:
            continue
        r = host[i]
        pos = 0
        for layer in range(L):
            kp[layer, b] = np.frombuffer(r[pos:pos + run].tobytes(), dtype=k_pool.dtype).reshape(tile)
            vp[layer, b] = np.frombuffer(r[pos + run:pos + 2 * run].tobytes(), dtype=v_pool.dtype).reshape(tile)
            pos += 2 * run
        if fp8:
            for layer in range(L):
                ks[layer, b] = np.frombuffer(r[pos:pos + 4 * H].tobytes(), dtype=np.float32)
                vs[layer, b] = np.frombuffer(r[pos + 4 * H:pos + 8 * H].tobytes(), dtype=np.float32)
                pos += 8 * H
    return (kp, vp, ks, vs) if fp8 else (kp, vp)
