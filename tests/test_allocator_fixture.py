"""The host block allocator used to build block tables (input fixture).

Contract from section 4 ("Minimal implementation") of the lattice-ai-eng
"KV Cache & PagedAttention" page: LIFO free list, MemoryError when empty,
reference counts raised by sharing and a block freed when its count reaches
zero, utilization as the fraction of blocks in use; plus the append rule that
a new block is taken only when the length is a multiple of B.
"""
import math

import numpy as np
import pytest

import kvgen


def test_lifo_exhaustion_and_refcounts():
    a = kvgen.BlockAllocator(4)
    got = [a.alloc() for _ in range(4)]
    assert got == [3, 2, 1, 0]
    assert a.utilization() == 1.0
    with pytest.raises(MemoryError):
        a.alloc()
    a.share(2)
    a.release(2)
    assert a.num_free() == 0          # still referenced once
    a.release(2)
    assert a.free == [2]
    assert a.alloc() == 2             # most recently freed block comes back first
    with pytest.raises(ValueError):
        a.release(7)


def test_shared_blocks_cost_nothing_until_released():
    a = kvgen.BlockAllocator(10)
    prefix = [a.alloc() for _ in range(3)]
    u = a.utilization()
    for _ in range(2):                 # two forks share the prefix
        for b in prefix:
            a.share(b)
    assert a.utilization() == u
    for b in prefix:
        assert a.refcount[b] == 3


def _grow(alloc, length, table, B):
    """Append one token; a new block only when the length is a multiple of B."""
    if length % B == 0:
        table.append(alloc.alloc())
    return length + 1


def test_append_rule_caps_waste_below_one_block():
    B = 16
    a = kvgen.BlockAllocator(1000)
    for L_final in (1, 15, 16, 17, 300, 301):
        table, L = [], 0
        for _ in range(L_final):
            L = _grow(a, L, table, B)
        assert len(table) == math.ceil(L_final / B)
        assert len(table) * B - L_final <= B - 1
        for b in table:
            a.release(b)


@pytest.mark.parametrize("name", ["C1", "C2", "C3", "C4", "C5"])
def test_generated_tables_are_consistent(name):
    wl = kvgen.make_workload(name, num_seqs=None if name in ("C1", "C5") else 16,
                             poison=True)
    B = wl.block_size
    seen = {}
    for i, L in enumerate(wl.context_lens):
        nb = math.ceil(int(L) / B)
        row = wl.block_tables[i, :nb]
        assert ((row >= 0) & (row < wl.num_blocks)).all()
        assert nb * B - int(L) <= B - 1
        for b in row:
            seen[int(b)] = seen.get(int(b), 0) + 1
    if name == "C4":
        shared = [b for b, c in seen.items() if c == wl.num_seqs]
        assert len(shared) == 128
    else:
        assert max(seen.values()) == 1   # private blocks only
    if name == "C5":
        assert wl.info["utilization"] == pytest.approx(0.8, abs=0.01)


def test_c1_shape_matches_its_description():
    wl = kvgen.make_workload("C1")
    assert list(wl.context_lens) == [17, 33, 100, 200]
    assert wl.num_blocks == 64 and wl.num_q_heads == 8 and wl.num_kv_heads == 2 and wl.head_dim == 64
    assert wl.dtype == "f32" and wl.num_write_tokens == 4


def test_c3_includes_the_prefill_chunk():
    wl = kvgen.make_workload("C3", num_seqs=8)
    assert wl.num_write_tokens == 8 + 2048
    assert wl.extra_tables.shape[0] == 1
    assert (wl.context_lens >= 16).all() and (wl.context_lens <= 8192).all()


def test_generation_is_deterministic():
    a = kvgen.make_workload("C2", num_seqs=3)
    b = kvgen.make_workload("C2", num_seqs=3)
    assert np.array_equal(a.k_pool, b.k_pool) and np.array_equal(a.block_tables, b.block_tables)
    assert np.array_equal(a.q, b.q)


def test_fork_then_append_copies_only_the_shared_tail_block():
    """n samples forked from one prompt cost one prompt plus n tails: only the
    partially filled tail block is copied, once per writer while it is still
    shared, and the last holder writes in place ("PagedAttention, Internals
    First", "03 Sharing via copy-on-write")."""
    B = 16
    alloc = kvgen.BlockAllocator(64)
    parent = [alloc.alloc() for _ in range(7)]          # a 100-token prompt: 6 full blocks + 4 tokens
    children = [alloc.fork(parent) for _ in range(3)]
    assert all(alloc.refcount[b] == 4 for b in parent)
    tail = parent[6]
    copies = []
    for row in children + [parent]:
        pair = alloc.cow_for_append(row, 100, B)
        if pair is not None:
            copies.append(pair)
    assert [src for src, _ in copies] == [tail] * 3     # three copies of the one tail block
    assert parent[6] == tail and alloc.refcount[tail] == 1
    assert len({row[6] for row in children + [parent]}) == 4
    assert all(alloc.refcount[b] == 4 for b in parent[:6])   # the full prompt blocks stay shared
    # next token of a child lands in its private block: no copy
    assert alloc.cow_for_append(children[0], 101, B) is None
    # a position that starts a new block takes a fresh one, no copy
    row = children[1]
    for pos in range(101, 112):
        assert alloc.cow_for_append(row, pos, B) is None
    assert alloc.cow_for_append(row, 112, B) is None and len(row) == 8


def test_full_prompt_blocks_never_copy():
    """A prompt that fills its last block leaves nothing to copy: every sample's
    first token opens a private block."""
    alloc = kvgen.BlockAllocator(300)
    parent = [alloc.alloc() for _ in range(125)]         # 2000 tokens = 125 full blocks
    rows = [alloc.fork(parent) for _ in range(3)] + [parent]
    assert all(alloc.cow_for_append(r, 2000, 16) is None for r in rows)
    assert all(len(r) == 126 for r in rows) and alloc.refcount[parent[0]] == 4
