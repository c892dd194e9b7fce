"""Seeded synthetic inputs for the paged KV-cache hot path.

This module is shared by the tests, the benchmark and the smoke check.  It
produces *inputs only*: element values, context lengths, block tables built by
a host block allocator, and the list of token positions each step writes.  It
holds none of the hot path's arithmetic: it never computes a slot index, never
scatters a token and never evaluates attention.  Both the HIP library and the
CPU oracle derive those from what is returned here.

Storage conventions (one layer, one K and one V tensor per layer, as the
"Sizing the pool" section of the aicassindra.com paged-KV-cache page states):

* ``k_pool`` / ``v_pool``: ``[num_blocks][num_kv_heads][block_size][head_dim]``
  with ``head_dim`` innermost and contiguous ("The write path: slot mapping and
  scatter" on the same page).  fp32 pools are ``numpy.float32``; bf16 pools are
  the raw 16-bit patterns as ``numpy.uint16``.
* ``q``: ``[num_seqs][num_q_heads][head_dim]``; ``k_new`` / ``v_new``:
  ``[num_tokens][num_kv_heads][head_dim]`` in the storage dtype.
* ``block_tables``: ``int32 [num_seqs][max_blocks_per_seq]``; entry ``b`` names
  the physical block of logical tokens ``[b*B, (b+1)*B)`` ("02 Block tables",
  PagedAttention, Internals First).
* ``context_lens``: ``int32 [num_seqs]``, counting the token written this step
  ("End-to-end flow" of the aicassindra.com transformer-math paged-attention
  page: the step attends over the full history including the new token).
* writes: ``write_seq`` / ``write_start`` / ``write_count`` (``int32``) name, per
  request, a table row and the run of logical positions whose K/V this step
  produces.  Decode requests write one position, ``context_lens[i] - 1``.
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional

import numpy as np

F32 = "f32"
BF16 = "bf16"

BF16_NAN = np.uint16(0x7FC0)
F32_NAN_BITS = np.uint32(0x7FC00000)

_CHUNK = 1 << 20  # elements per independently seeded chunk (fixed => deterministic)


# ----------------------------------------------------------------------------
# value generation
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); NaN stays NaN."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = BF16_NAN
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal_fill(shape, seed_seq: np.random.SeedSequence, scale: float, dtype: str) -> np.ndarray:
    """N(0, scale^2) values in the storage dtype, filled in fixed seeded chunks.

    Every chunk of ``_CHUNK`` elements draws from its own child of ``seed_seq``,
    so the result does not depend on the thread count.
    """
    n = int(np.prod(shape))
    nchunks = max(1, (n + _CHUNK - 1) // _CHUNK)
    kids = seed_seq.spawn(nchunks)
    res = np.empty(n, dtype=np.float32 if dtype == F32 else np.uint16)

    def work(i):
        lo, hi = i * _CHUNK, min(n, (i + 1) * _CHUNK)
        g = np.random.default_rng(kids[i])
        if dtype == F32:
            g.standard_normal(out=res[lo:hi], dtype=np.float32)
            if scale != 1.0:
                res[lo:hi] *= np.float32(scale)
            return
        buf = np.empty(hi - lo, dtype=np.float32)
        g.standard_normal(out=buf, dtype=np.float32)
        if scale != 1.0:
            buf *= np.float32(scale)
        # round to nearest even bfloat16, in place on the bit pattern (no NaN here)
        u = buf.view(np.uint32)
        odd = (u >> np.uint32(16)) & np.uint32(1)
        u += np.uint32(0x7FFF)
        u += odd
        u >>= np.uint32(16)
        res[lo:hi] = u

    if nchunks == 1:
        work(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nchunks)))
    return res.reshape(shape)


def nan_value(dtype: str):
    return np.float32(np.nan) if dtype == F32 else BF16_NAN


# ----------------------------------------------------------------------------
# host block allocator fixture
# ----------------------------------------------------------------------------

class BlockAllocator:
    """Block manager fixture: which physical blocks are free and how many
    tables name each of the others.

    State is two arrays: ``_stack[:_top]`` holds the free block ids (the next
    block handed out is ``_stack[_top - 1]``, and a released block goes back
    on top, so the most recently freed block is reused first, as a LIFO free
    list does), and ``_refs[b]`` counts the tables naming block ``b`` (0 for a
    free block).  The behaviour is the block manager's contract as the pages
    state it (lattice-ai-eng "KV Cache & PagedAttention", section 4; "GPU
    paged KV cache", "Prefix sharing, reference counts, and copy-on-write"):
    an empty pool is a ``MemoryError`` for the caller, sharing adds a
    reference, a block returns to the pool when its last reference goes, and
    utilization is the fraction of blocks in use.
    """

    def __init__(self, num_blocks: int, order: Optional[np.ndarray] = None):
        n = int(num_blocks)
        ids = np.arange(n, dtype=np.int64) if order is None else np.asarray(order, dtype=np.int64).reshape(-1)
        if ids.shape != (n,) or not np.array_equal(np.sort(ids), np.arange(n)):
            raise ValueError("free-list order must be a permutation of the pool")
        self.num_blocks = n
        self._stack = ids.astype(np.int32)
        self._top = n
        self._refs = np.zeros(n, dtype=np.int32)

    def _held(self, b: int, what: str) -> int:
        b = int(b)
        if not 0 <= b < self.num_blocks or self._refs[b] <= 0:
            raise ValueError(f"{what} of block {b} that holds no reference")
        return b

    def alloc(self) -> int:
        if self._top == 0:
            raise MemoryError("KV block pool exhausted")
        self._top -= 1
        b = int(self._stack[self._top])
        self._refs[b] = 1
        return b

    def release(self, b: int) -> None:
        b = self._held(b, "release")
        self._refs[b] -= 1
        if self._refs[b] == 0:
            self._stack[self._top] = b
            self._top += 1

    def share(self, b: int) -> int:
        b = self._held(b, "share")
        self._refs[b] += 1
        return b

    @property
    def free(self) -> List[int]:
        """Free blocks, the next to be handed out last."""
        return [int(b) for b in self._stack[:self._top]]

    @property
    def refcount(self) -> Dict[int, int]:
        """References of every block in use (a snapshot)."""
        held = np.flatnonzero(self._refs)
        return {int(b): int(self._refs[b]) for b in held}

    def fork(self, row) -> List[int]:
        """A child table naming the same blocks (every count goes up by one)."""
        return [self.share(int(b)) for b in row]

    def cow_for_append(self, row: List[int], pos: int, block_size: int):
        """The refcount check on the append path ("PagedAttention, Internals
        First", "03 Sharing via copy-on-write"; aicassindra.com "GPU paged KV
        cache", "Prefix sharing, reference counts, and copy-on-write").

        Token ``pos`` of the sequence whose table is ``row`` is about to be
        written.  A fresh block is appended when ``pos`` starts a new block.
        If its block is named by more than one table, a fresh block is taken,
        the old count goes down by one and ``row`` is repointed; the
        ``(src, dst)`` pair of the device copy is returned.  Otherwise (count
        1: write in place) ``None``.
        """
        b = pos // block_size
        if b == len(row):
            row.append(self.alloc())
            return None
        old = int(row[b])
        if self._refs[old] > 1:
            new = self.alloc()
            self.release(old)
            row[b] = new
            return (old, new)
        return None

    def num_free(self) -> int:
        return self._top

    def utilization(self) -> float:
        return 1.0 - self._top / self.num_blocks if self.num_blocks else 0.0


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class Workload:
    name: str
    variant: str
    dtype: str
    num_blocks: int
    block_size: int
    num_kv_heads: int
    num_q_heads: int
    head_dim: int
    context_lens: np.ndarray          # int32 [S]
    block_tables: np.ndarray          # int32 [S][MB]
    write_seq: np.ndarray             # int32 [R]
    write_start: np.ndarray           # int32 [R]
    write_count: np.ndarray           # int32 [R]
    extra_tables: np.ndarray          # int32 [E][MB] rows that only receive writes (prefill)
    q: np.ndarray                     # [S][Hq][D]
    k_new: np.ndarray                 # [T][Hkv][D]
    v_new: np.ndarray                 # [T][Hkv][D]
    k_pool: np.ndarray                # [N][Hkv][B][D] before the step's writes
    v_pool: np.ndarray
    partition_size: int = 0
    refcounts: Optional[Dict[int, int]] = None
    info: Dict[str, object] = dataclasses.field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def num_write_tokens(self) -> int:
        return int(self.write_count.sum())

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == F32 else 2

    def all_tables(self) -> np.ndarray:
        """Decode rows followed by write-only rows: the table the write requests index."""
        if self.extra_tables.shape[0] == 0:
            return self.block_tables
        return np.concatenate([self.block_tables, self.extra_tables], axis=0)


def _blocks_for(n_tokens: int, B: int) -> int:
    return -(-int(n_tokens) // B)


@dataclasses.dataclass
class Shape:
    name: str
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    value_scale: float
    partition_size: int = 0


def _lengths(name: str, rng: np.random.Generator, S: int) -> np.ndarray:
    if name == "C1":
        return np.array([17, 33, 100, 200], dtype=np.int32)[:S]
    if name == "C2":
        return rng.integers(512, 4096, size=S, endpoint=True).astype(np.int32)
    if name == "C3":
        # lognormal with median 1024; sigma is not given on the pages: 1.0 is the reading taken
        x = rng.lognormal(mean=math.log(1024.0), sigma=1.0, size=S)
        return np.clip(np.rint(x), 16, 8192).astype(np.int32)
    if name == "C4":
        return (2048 + rng.integers(64, 512, size=S, endpoint=True)).astype(np.int32)
    if name == "C5":
        return rng.integers(32768, 131072, size=S, endpoint=True).astype(np.int32)
    raise ValueError(name)


CONFIGS = {
    # tiny fp32 case
    "C1": dict(S=4, shape=Shape("C1", F32, 8, 2, 64, 16, 1.0)),
    # Llama-3-8B-shaped decode layer
    "C2": dict(S=64, shape=Shape("C2", BF16, 32, 8, 128, 16, 1.0 / math.sqrt(128))),
    # 70B-class GQA decode layer plus a 2048-token prefill chunk scatter
    "C3": dict(S=256, shape=Shape("C3", BF16, 64, 8, 128, 16, 1.0 / math.sqrt(128))),
    # prefix-sharing decode
    "C4": dict(S=128, shape=Shape("C4", BF16, 32, 8, 128, 16, 1.0 / math.sqrt(128))),
    # long-context decode, split into 512-token partitions
    "C5": dict(S=8, shape=Shape("C5", BF16, 32, 8, 128, 16, 1.0 / math.sqrt(128), partition_size=512)),
    # one GPU's share of the 70B-class layer under tensor parallelism over KV
    # heads at TP = 8 (each GPU holds H_kv / 8 KV heads and their H_q / 8 query
    # heads): the same batch as C3 (same seed: same lengths, tables and
    # prefill chunk) with 8 query heads and 1 KV head
    "C3TP8": dict(S=256, shape=Shape("C3", BF16, 8, 1, 128, 16, 1.0 / math.sqrt(128)), base="C3", seed=3),
}

VARIANTS = ("spec", "sharp", "hot", "needle")


def make_workload(name: str, seed: Optional[int] = None, variant: str = "spec", *,
                  num_seqs: Optional[int] = None, poison: bool = False,
                  unshared: bool = False, lengths: Optional[np.ndarray] = None,
                  shape: Optional[Shape] = None, num_blocks: Optional[int] = None,
                  table_pad: int = 0, block_size: Optional[int] = None) -> Workload:
    """Build one seeded workload.

    name     one of C1..C5 (or any name when ``shape`` and ``lengths`` are given)
    seed     defaults to the config number (C1 -> 1, ...)
    variant  value distribution: "spec" as specified, "sharp" unscaled N(0,1),
             "hot" unscaled with Q x 30 (logits of order 100), "needle" unscaled
             plus one key per (sequence, KV head) aligned with a query head
    num_seqs override the batch size (smaller parity cases)
    poison   NaN in every slot that no table entry covers below the context
             length (stale slots, unreferenced blocks, the slot about to be
             written) and unused table entries pointed at a NaN block
    """
    if variant not in VARIANTS:
        raise ValueError(f"unknown variant {variant}")
    cfg = CONFIGS.get(name)
    if shape is None:
        if cfg is None:
            raise ValueError(f"unknown config {name}")
        shape = cfg["shape"]
    if block_size is not None:
        shape = dataclasses.replace(shape, block_size=int(block_size))
    base = cfg.get("base", name) if cfg else name   # the configuration whose batch this one is
    if seed is None:
        seed = cfg["seed"] if cfg and "seed" in cfg else (int(name[1:]) if name[1:].isdigit() else 0)
    S = num_seqs if num_seqs is not None else (cfg["S"] if cfg else len(lengths))
    B, Hkv, Hq, D, dt = shape.block_size, shape.num_kv_heads, shape.num_q_heads, shape.head_dim, shape.dtype
    ss = np.random.SeedSequence([seed, VARIANTS.index(variant), 1 if poison else 0])
    ss_len, ss_tab, ss_q, ss_k, ss_v, ss_pool_k, ss_pool_v, ss_needle = ss.spawn(8)
    rng_len = np.random.default_rng(ss_len)
    rng_tab = np.random.default_rng(ss_tab)

    if lengths is None:
        lengths = _lengths(shape.name if cfg is None else base, rng_len, S)
    lengths = np.asarray(lengths, dtype=np.int32)
    S = int(lengths.shape[0])
    nblk = np.array([_blocks_for(L, B) for L in lengths], dtype=np.int64)
    info: Dict[str, object] = {}
    extra_rows: List[List[int]] = []
    refcounts = None

    # ---------------- block tables -------------------------------------
    tables_rows: List[List[int]] = []
    if name == "C1" and num_blocks is None:
        N = 64
        perm = rng_tab.permutation(N)
        pos = 0
        for i in range(S):
            tables_rows.append([int(b) for b in perm[pos:pos + nblk[i]]])
            pos += int(nblk[i])
    elif name == "C4" and cfg is not None:
        prefix_tokens = 2048
        n_prefix = prefix_tokens // B
        private = [int(n) - n_prefix for n in nblk]
        need = n_prefix + sum(private)
        N = num_blocks or int(math.ceil(1.25 * need))
        alloc = BlockAllocator(N, rng_tab.permutation(N))
        shared = [alloc.alloc() for _ in range(n_prefix)]
        for i in range(S):
            row = [alloc.share(b) for b in shared] if i > 0 else list(shared)
            row += [alloc.alloc() for _ in range(private[i])]
            tables_rows.append(row)
        refcounts = dict(alloc.refcount)
        info["shared_prefix_blocks"] = n_prefix
        info["utilization"] = alloc.utilization()
    elif name == "C5" and cfg is not None:
        need = int(nblk.sum())
        N = num_blocks or int(math.ceil(1.25 * need))
        alloc = BlockAllocator(N, rng_tab.permutation(N))
        # churn: 10k seeded alloc/free cycles over dummy sequences, then release them all
        dummies: List[List[int]] = []
        for _ in range(10_000):
            if rng_tab.random() < 0.5:
                k = int(rng_tab.integers(1, 64, endpoint=True))
                if alloc.num_free() >= k:
                    dummies.append([alloc.alloc() for _ in range(k)])
            elif dummies:
                j = int(rng_tab.integers(0, len(dummies)))
                for b in dummies.pop(j):
                    alloc.release(b)
        for d in dummies:
            for b in d:
                alloc.release(b)
        # real sequences grow block by block, round-robin, as decode growth would
        tables_rows = [[] for _ in range(S)]
        for step in range(int(nblk.max())):
            for i in range(S):
                if step < nblk[i]:
                    tables_rows[i].append(alloc.alloc())
        info["utilization"] = alloc.utilization()
    else:
        prefill = 2048 if (base == "C3" and cfg is not None) else 0
        need = int(nblk.sum())
        N = num_blocks or max(1, int(math.ceil(1.25 * need))) + prefill // B
        alloc = BlockAllocator(N, rng_tab.permutation(N))
        for i in range(S):
            tables_rows.append([alloc.alloc() for _ in range(int(nblk[i]))])
        if prefill:
            extra_rows.append([alloc.alloc() for _ in range(prefill // B)])
        info["utilization"] = alloc.utilization()

    MB = max([len(r) for r in tables_rows + extra_rows] + [1]) + table_pad
    used = np.zeros(N, dtype=bool)
    for r in tables_rows + extra_rows:
        used[r] = True
    unref = np.flatnonzero(~used)
    fill = int(unref[0]) if (poison and unref.size) else 0
    tables = np.full((S, MB), fill, dtype=np.int32)
    for i, r in enumerate(tables_rows):
        tables[i, :len(r)] = r
    extra = np.full((len(extra_rows), MB), fill, dtype=np.int32)
    for i, r in enumerate(extra_rows):
        extra[i, :len(r)] = r

    # ---------------- write requests -----------------------------------
    wseq = list(range(S))
    wstart = [int(L) - 1 for L in lengths]
    wcount = [1] * S
    for j, r in enumerate(extra_rows):
        wseq.append(S + j)
        wstart.append(0)
        wcount.append(len(r) * B)
    keep = [k for k in range(len(wseq)) if wcount[k] > 0 and wstart[k] >= 0]
    write_seq = np.array([wseq[k] for k in keep], dtype=np.int32)
    write_start = np.array([wstart[k] for k in keep], dtype=np.int32)
    write_count = np.array([wcount[k] for k in keep], dtype=np.int32)
    T = int(write_count.sum())

    # ---------------- values -------------------------------------------
    scale = shape.value_scale if variant == "spec" else 1.0
    q = normal_fill((S, Hq, D), ss_q, scale * (30.0 if variant == "hot" else 1.0), dt)
    k_new = normal_fill((T, Hkv, D), ss_k, scale, dt)
    v_new = normal_fill((T, Hkv, D), ss_v, scale, dt)
    k_pool = normal_fill((N, Hkv, B, D), ss_pool_k, scale, dt)
    v_pool = normal_fill((N, Hkv, B, D), ss_pool_v, scale, dt)

    if variant == "needle":
        # One key per (sequence, KV head) is set to 4x the first query head of
        # its group, at a position that cycles through the first token, the
        # token written this step, the last full block and partition edges.
        rng_n = np.random.default_rng(ss_needle)
        g = Hq // Hkv
        tok_of_req = {}
        t0 = 0
        for k in range(len(write_seq)):
            if write_seq[k] < S and write_count[k] == 1:
                tok_of_req[int(write_seq[k])] = t0
            t0 += int(write_count[k])
        P = shape.partition_size or 512
        for i in range(S):
            L = int(lengths[i])
            if L <= 0:
                continue
            choices = [0, L - 1, max(0, (L // B) * B - 1), min(L - 1, P - 1), min(L - 1, P),
                       int(rng_n.integers(0, L))]
            pos = choices[i % len(choices)]
            for kv in range(Hkv):
                h = kv * g
                if dt == F32:
                    val = (4.0 * q[i, h].astype(np.float32))
                    vbits = val
                else:
                    val = 4.0 * bf16_bits_to_f32(q[i, h])
                    vbits = f32_to_bf16_bits(val)
                if pos == L - 1 and i in tok_of_req:
                    k_new[tok_of_req[i], kv] = vbits
                else:
                    blk = tables_rows[i][pos // B]
                    k_pool[blk, kv, pos % B] = vbits
        info["needle"] = True

    if poison:
        nanv = nan_value(dt)
        # unreferenced blocks
        k_pool[unref] = nanv
        v_pool[unref] = nanv
        # stale slots at and past the position written this step, in each row's last block
        for i, r in enumerate(tables_rows):
            L = int(lengths[i])
            if not r:
                continue
            first_stale = L - 1 if L > 0 else 0
            for pos in range(first_stale, len(r) * B):
                blk = r[pos // B]
                # a shared block can hold another sequence's live tokens: never poison those
                if refcounts and refcounts.get(blk, 1) > 1:
                    continue
                k_pool[blk, :, pos % B] = nanv
                v_pool[blk, :, pos % B] = nanv
        for r in extra_rows:
            for blk in r:
                k_pool[blk] = nanv
                v_pool[blk] = nanv
        info["poison"] = True

    info["seed"] = seed
    if base == "C3":
        info["lognormal_sigma"] = 1.0
    return Workload(name=name, variant=variant, dtype=dt, num_blocks=N, block_size=B,
                    num_kv_heads=Hkv, num_q_heads=Hq, head_dim=D,
                    context_lens=lengths, block_tables=tables,
                    write_seq=write_seq, write_start=write_start, write_count=write_count,
                    extra_tables=extra, q=q, k_new=k_new, v_new=v_new,
                    k_pool=k_pool, v_pool=v_pool, partition_size=shape.partition_size,
                    refcounts=refcounts, info=info)


def custom_workload(*, lengths, num_q_heads: int, num_kv_heads: int, head_dim: int,
                    dtype: str, block_size: int = 16, seed: int = 0, variant: str = "sharp",
                    poison: bool = True, num_blocks: Optional[int] = None,
                    table_pad: int = 0, partition_size: int = 0) -> Workload:
    """A workload with explicit lengths and head shape (ragged and edge cases)."""
    shape = Shape("custom", dtype, num_q_heads, num_kv_heads, head_dim, block_size, 1.0,
                  partition_size=partition_size)
    return make_workload("custom", seed=seed, variant=variant, poison=poison,
                         lengths=np.asarray(lengths, dtype=np.int32), shape=shape,
                         num_blocks=num_blocks, table_pad=table_pad)


# ----------------------------------------------------------------------------
# relayouts of an existing workload (same logical contents, other physical blocks)
# ----------------------------------------------------------------------------

def _rebuild(wl: Workload, new_tables: np.ndarray, new_extra: np.ndarray,
             k_pool: np.ndarray, v_pool: np.ndarray, tag: str) -> Workload:
    out = dataclasses.replace(wl, block_tables=new_tables, extra_tables=new_extra,
                              k_pool=k_pool, v_pool=v_pool, num_blocks=int(k_pool.shape[0]),
                              refcounts=None, info=dict(wl.info, relayout=tag))
    return out


def permute_blocks(wl: Workload, seed: int) -> Workload:
    """Move every physical block to a new index given by a seeded permutation.

    Block contents travel with their block, and the tables are renamed to
    match, so every sequence sees the same logical K/V.
    """
    N = wl.num_blocks
    perm = np.random.default_rng(seed).permutation(N)   # old index -> new index
    k = np.empty_like(wl.k_pool)
    v = np.empty_like(wl.v_pool)
    k[perm] = wl.k_pool
    v[perm] = wl.v_pool
    return _rebuild(wl, perm[wl.block_tables].astype(np.int32),
                    perm[wl.extra_tables].astype(np.int32) if wl.extra_tables.size else wl.extra_tables,
                    k, v, "permuted")


def _used_rows(wl: Workload):
    rows = []
    for i in range(wl.num_seqs):
        n = _blocks_for(int(wl.context_lens[i]), wl.block_size)
        rows.append([int(b) for b in wl.block_tables[i, :n]])
    extra = []
    for r in range(wl.extra_tables.shape[0]):
        k = [k for k in range(len(wl.write_seq)) if wl.write_seq[k] == wl.num_seqs + r][0]
        n = _blocks_for(int(wl.write_start[k]) + int(wl.write_count[k]), wl.block_size)
        extra.append([int(b) for b in wl.extra_tables[r, :n]])
    return rows, extra


def privatize_blocks(wl: Workload, *, contiguous: bool = False) -> Workload:
    """Give every table entry its own physical block holding a copy of the old one.

    With ``contiguous`` the copies of sequence i are laid out back to back in
    logical order (block-table rows become 0,1,2,... ranges): the dense layout a
    contiguous cache would have.  Otherwise the copies keep the original
    relative order of first use.  Blocks referenced by no table are dropped,
    except one NaN-filled spare that unused table entries point at.
    """
    rows, extra = _used_rows(wl)
    src = [b for r in rows + extra for b in r]
    n_new = len(src) + 1
    spare = n_new - 1
    k = np.empty((n_new,) + wl.k_pool.shape[1:], dtype=wl.k_pool.dtype)
    v = np.empty_like(k)
    k[:len(src)] = wl.k_pool[src]
    v[:len(src)] = wl.v_pool[src]
    k[spare] = nan_value(wl.dtype)
    v[spare] = nan_value(wl.dtype)
    tables = np.full_like(wl.block_tables, spare)
    pos = 0
    for i, r in enumerate(rows):
        tables[i, :len(r)] = np.arange(pos, pos + len(r))
        pos += len(r)
    ext = np.full_like(wl.extra_tables, spare)
    for i, r in enumerate(extra):
        ext[i, :len(r)] = np.arange(pos, pos + len(r))
        pos += len(r)
    return _rebuild(wl, tables, ext, k, v, "contiguous" if contiguous else "private")


# ----------------------------------------------------------------------------
# FP8 pool contents (codes and block scales as stored, drawn directly)
# ----------------------------------------------------------------------------

E4M3_NAN_CODE = np.uint8(0x7F)
# the 254 byte values that are finite E4M3 codes (0x7F and 0xFF are NaN)
FINITE_E4M3_CODES = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)


def fp8_codes(shape, seed_seq: np.random.SeedSequence) -> np.ndarray:
    """Codes drawn uniformly from the finite E4M3 codes, so every exponent,
    both signs, zeros and subnormals occur."""
    n = int(np.prod(shape))
    nchunks = max(1, (n + _CHUNK - 1) // _CHUNK)
    kids = seed_seq.spawn(nchunks)
    res = np.empty(n, dtype=np.uint8)

    def work(i):
        lo, hi = i * _CHUNK, min(n, (i + 1) * _CHUNK)
        g = np.random.default_rng(kids[i])
        res[lo:hi] = FINITE_E4M3_CODES[g.integers(0, FINITE_E4M3_CODES.size, size=hi - lo)]

    if nchunks == 1:
        work(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nchunks)))
    return res.reshape(shape)


def fp8_pool_state(wl: Workload, *, seed: int = 0, largest: float = 3.0, spread: float = 0.1):
    """An FP8 pool with the block layout of ``wl``: (k_codes, v_codes, k_scale,
    v_scale), codes ``uint8 [N][Hkv][B][D]``, scales ``float32 [N][Hkv]``.

    Codes are uniform over the finite codes; scales are lognormal with median
    ``largest / 448`` (the largest code then stands for about ``largest``,
    the magnitude of the largest of 128 N(0, 1) values) and log-spread
    ``spread``.  Wherever ``wl`` holds a NaN stale slot (a poisoned workload),
    the code is NaN (0x7F) too.
    """
    ss = np.random.SeedSequence([seed, 8])
    s_kc, s_vc, s_ks, s_vs = ss.spawn(4)
    N, H, B, D = wl.k_pool.shape
    kc = fp8_codes((N, H, B, D), s_kc)
    vc = fp8_codes((N, H, B, D), s_vc)
    med = math.log(largest / 448.0)
    ks = np.exp(np.random.default_rng(s_ks).normal(med, spread, size=(N, H))).astype(np.float32)
    vs = np.exp(np.random.default_rng(s_vs).normal(med, spread, size=(N, H))).astype(np.float32)
    if wl.dtype == BF16:
        bits = wl.k_pool.view(np.uint16)
        stale = (bits & np.uint16(0x7FFF)) > np.uint16(0x7F80)
    else:
        stale = np.isnan(wl.k_pool)
    kc[stale] = E4M3_NAN_CODE
    vc[stale] = E4M3_NAN_CODE
    return kc, vc, ks, vs
