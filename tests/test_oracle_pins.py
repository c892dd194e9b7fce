"""Pins for the CPU oracle: checks against things other than the oracle itself.

* a library routine: on a contiguous layout, paged attention must equal
  ``torch.nn.functional.scaled_dot_product_attention`` in fp64 with the KV
  heads repeated over their query-head groups (paging is invisible to the
  math: aicassindra.com transformer-math paged attention, "The architecture:
  every piece explained"; KV Cache & PagedAttention, section 5: lossless);
* closed forms (one token, zero query, needle key);
* invariances the pages state (physical placement is arbitrary: "02 Block
  tables" of PagedAttention, Internals First; reads do not care about
  sharing: its section 03);
* the scatter as a byte copy (aicassindra.com GPU paged KV cache, "The write
  path: slot mapping and scatter") and the slot formula;
* negative controls: the comparison used by the parity tests must reject
  plausible wrong answers.
"""
import math

import numpy as np
import pytest
import torch

import kvgen
import oracle


def _to_f64(a, dtype):
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    return kvgen.bf16_bits_to_f32(a).astype(np.float64)


def _sdpa_reference(wl, k_pool, v_pool, scale, interleave=True):
    """Library attention on the dense layout of each sequence.

    ``privatize_blocks(contiguous=True)`` lays each sequence's blocks out back
    to back, so its K for KV head h is rows [start, start+L) of the
    [num_blocks][H][B][D] pool read as [H][blocks*B][D].
    """
    dense = kvgen.privatize_blocks(kvgen.dataclasses.replace(wl, k_pool=k_pool, v_pool=v_pool),
                                   contiguous=True)
    g = wl.num_q_heads // wl.num_kv_heads
    outs = np.zeros((wl.num_seqs, wl.num_q_heads, wl.head_dim))
    for i in range(wl.num_seqs):
        L = int(wl.context_lens[i])
        if L == 0:
            continue
        nb = -(-L // wl.block_size)
        first = int(dense.block_tables[i, 0])
        assert list(dense.block_tables[i, :nb]) == list(range(first, first + nb))
        kk = _to_f64(dense.k_pool[first:first + nb], wl.dtype)      # [nb][H][B][D]
        vv = _to_f64(dense.v_pool[first:first + nb], wl.dtype)
        K = torch.from_numpy(kk.transpose(1, 0, 2, 3).reshape(wl.num_kv_heads, nb * wl.block_size, wl.head_dim)[:, :L])
        V = torch.from_numpy(vv.transpose(1, 0, 2, 3).reshape(wl.num_kv_heads, nb * wl.block_size, wl.head_dim)[:, :L])
        if interleave:   # query head h reads KV head h // g
            K = K.repeat_interleave(g, dim=0).contiguous()
            V = V.repeat_interleave(g, dim=0).contiguous()
        else:            # the other plausible mapping, h % H_kv
            K = K.repeat(g, 1, 1).contiguous()
            V = V.repeat(g, 1, 1).contiguous()
        Q = torch.from_numpy(_to_f64(wl.q[i], wl.dtype)).unsqueeze(1)   # [Hq][1][D]
        o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=scale)
        outs[i] = o[:, 0].numpy()
    return outs


SHAPES = [
    # (dtype, Hq, Hkv, D, lengths)
    ("f32", 8, 2, 64, [17, 33, 100, 200]),
    ("bf16", 32, 8, 128, [1, 16, 47, 300]),
    ("bf16", 8, 1, 64, [5, 64, 129]),
    ("f32", 4, 4, 128, [2, 31, 77]),
    ("bf16", 64, 8, 128, [16, 40, 301]),
]


@pytest.mark.parametrize("dtype,hq,hkv,d,lengths", SHAPES)
def test_attention_equals_library_sdpa(dtype, hq, hkv, d, lengths):
    wl = kvgen.custom_workload(lengths=lengths, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                               dtype=dtype, seed=11, variant="sharp", poison=True)
    scale = 1.0 / math.sqrt(d)
    r = oracle.run_step(wl, scale=scale)
    ref = _sdpa_reference(wl, r["k_pool"], r["v_pool"], scale)
    assert np.isfinite(r["out"]).all()
    np.testing.assert_allclose(r["out"], ref, rtol=0, atol=1e-12)


def test_scale_argument_is_used():
    wl = kvgen.custom_workload(lengths=[50, 90], num_q_heads=4, num_kv_heads=2, head_dim=64,
                               dtype="f32", seed=3, variant="sharp")
    r = oracle.run_step(wl, scale=0.37)
    ref = _sdpa_reference(wl, r["k_pool"], r["v_pool"], 0.37)
    np.testing.assert_allclose(r["out"], ref, rtol=0, atol=1e-12)
    r2 = oracle.run_step(wl, scale=0.125)
    assert np.abs(r2["out"] - r["out"]).max() > 1e-3


def test_gqa_group_mapping_is_consecutive():
    """Query head h reads KV head h // g; h % H_kv would fail the library check."""
    wl = kvgen.custom_workload(lengths=[40, 70], num_q_heads=8, num_kv_heads=2, head_dim=64,
                               dtype="f32", seed=5, variant="sharp")
    r = oracle.run_step(wl)
    ref = _sdpa_reference(wl, r["k_pool"], r["v_pool"], 1 / 8)
    np.testing.assert_allclose(r["out"], ref, atol=1e-12)
    # the library with the other mapping (h % H_kv) differs clearly
    wrong = _sdpa_reference(wl, r["k_pool"], r["v_pool"], 1 / 8, interleave=False)
    assert np.abs(wrong - r["out"]).max() > 1e-1


def test_single_token_returns_its_value_exactly():
    for dtype in ("f32", "bf16"):
        wl = kvgen.custom_workload(lengths=[1, 1, 1], num_q_heads=4, num_kv_heads=2, head_dim=128,
                                   dtype=dtype, seed=7, variant="hot")
        r = oracle.run_step(wl)
        v = _to_f64(wl.v_new, dtype)  # the one token is the one written this step
        g = 2
        for i in range(3):
            for h in range(4):
                assert np.array_equal(r["out"][i, h], v[i, h // g])


def test_zero_query_gives_mean_of_values():
    wl = kvgen.custom_workload(lengths=[37, 64, 200], num_q_heads=2, num_kv_heads=1, head_dim=64,
                               dtype="bf16", seed=9, variant="sharp")
    wl.q[...] = 0
    r = oracle.run_step(wl)
    for i, L in enumerate(wl.context_lens):
        nb = -(-int(L) // 16)
        rows = []
        for j in range(int(L)):
            rows.append(_to_f64(r["v_pool"][wl.block_tables[i, j // 16], 0, j % 16], "bf16"))
        mean = np.mean(np.stack(rows), axis=0)
        np.testing.assert_allclose(r["out"][i, 0], mean, atol=1e-13)
        np.testing.assert_allclose(r["out"][i, 1], mean, atol=1e-13)


def test_needle_selects_its_value():
    wl = kvgen.custom_workload(lengths=[100, 33], num_q_heads=1, num_kv_heads=1, head_dim=64,
                               dtype="f32", seed=2, variant="sharp", poison=False)
    # key at logical position 70 of sequence 0 (block 4, offset 6) made parallel to q, large
    blk = wl.block_tables[0, 70 // 16]
    wl.k_pool[blk, 0, 70 % 16] = 50.0 * wl.q[0, 0] / np.linalg.norm(wl.q[0, 0])
    r = oracle.run_step(wl)
    np.testing.assert_allclose(r["out"][0, 0], wl.v_pool[blk, 0, 70 % 16].astype(np.float64), atol=1e-9)


def test_physical_permutation_invariance_is_exact():
    wl = kvgen.make_workload("C1", variant="sharp", poison=True)
    a = oracle.run_step(wl)["out"]
    for s in (1, 2, 3):
        b = oracle.run_step(kvgen.permute_blocks(wl, s))["out"]
        assert np.array_equal(a, b)


def test_shared_prefix_equals_private_copies_exactly():
    wl = kvgen.make_workload("C4", variant="sharp", num_seqs=6)
    assert wl.refcounts is not None and max(wl.refcounts.values()) == 6
    a = oracle.run_step(wl)["out"]
    b = oracle.run_step(kvgen.privatize_blocks(wl))["out"]
    assert np.array_equal(a, b)


def test_stale_slots_are_never_read():
    wl = kvgen.make_workload("C1", variant="sharp", poison=True)
    a = oracle.run_step(wl)["out"]
    assert np.isfinite(a).all()
    clean = kvgen.dataclasses.replace(wl, k_pool=np.nan_to_num(wl.k_pool), v_pool=np.nan_to_num(wl.v_pool))
    b = oracle.run_step(clean)["out"]
    assert np.array_equal(a, b)


def test_zero_length_gives_zero_output():
    wl = kvgen.custom_workload(lengths=[0, 20], num_q_heads=2, num_kv_heads=1, head_dim=64,
                               dtype="f32", seed=1)
    r = oracle.run_step(wl)
    assert np.array_equal(r["out"][0], np.zeros((2, 64)))
    assert np.isfinite(r["out"][1]).all()


def test_thread_count_does_not_change_result():
    wl = kvgen.make_workload("C2", variant="sharp", num_seqs=5)
    a = oracle.run_step(wl, threads=1)["out"]
    b = oracle.run_step(wl, threads=7)["out"]
    assert np.array_equal(a, b)


# ---------------------------------------------------------------- scatter --

def test_scatter_is_a_byte_copy_and_touches_nothing_else():
    for name in ("C1", "C3"):
        wl = kvgen.make_workload(name, variant="sharp", poison=True,
                                 num_seqs=None if name == "C1" else 12)
        slots = oracle.slot_mapping(wl.all_tables(), wl.block_size, wl.num_blocks,
                                    wl.write_seq, wl.write_start, wl.write_count)
        kp, vp = oracle.scatter(wl.k_pool, wl.v_pool, wl.k_new, wl.v_new, slots)
        B = wl.block_size
        touched = np.zeros((wl.num_blocks, B), dtype=bool)
        for t, s in enumerate(slots):
            blk, off = divmod(int(s), B)
            touched[blk, off] = True
            # round trip: the slot holds exactly the token's bits, every head
            assert kp[blk, :, off].tobytes() == wl.k_new[t].tobytes()
            assert vp[blk, :, off].tobytes() == wl.v_new[t].tobytes()
        untouched = ~touched
        a = kp.transpose(0, 2, 1, 3)[untouched].view(np.uint8)
        b = wl.k_pool.transpose(0, 2, 1, 3)[untouched].view(np.uint8)
        assert np.array_equal(a, b)
        a = vp.transpose(0, 2, 1, 3)[untouched].view(np.uint8)
        b = wl.v_pool.transpose(0, 2, 1, 3)[untouched].view(np.uint8)
        assert np.array_equal(a, b)


def test_scatter_skips_negative_slots():
    wl = kvgen.make_workload("C1", variant="sharp")
    slots = np.array([-1, -5, -1, -1], dtype=np.int64)
    kp, vp = oracle.scatter(wl.k_pool, wl.v_pool, wl.k_new, wl.v_new, slots)
    assert kp.tobytes() == wl.k_pool.tobytes() and vp.tobytes() == wl.v_pool.tobytes()


def test_c1_writes_land_at_block_starts_and_mid_block():
    """C1's lengths 17, 33, 100, 200 put the new token at offsets 0, 0, 3, 7."""
    wl = kvgen.make_workload("C1")
    slots = oracle.slot_mapping(wl.all_tables(), 16, wl.num_blocks, wl.write_seq,
                                wl.write_start, wl.write_count)
    expect_logical = [(1, 0), (2, 0), (6, 3), (12, 7)]
    for i, (lb, off) in enumerate(expect_logical):
        assert slots[i] == wl.block_tables[i, lb] * 16 + off


def test_slot_mapping_rejects_out_of_table_positions():
    tables = np.array([[3, 1]], dtype=np.int32)
    with pytest.raises(ValueError):
        oracle.slot_mapping(tables, 16, 4, np.array([0]), np.array([32]), np.array([1]))
    with pytest.raises(ValueError):
        oracle.slot_mapping(np.array([[9]], dtype=np.int32), 16, 4, np.array([0]), np.array([0]), np.array([1]))


# ------------------------------------------------------ negative controls --

def _bf16_gate(got, ref):
    return float(np.abs(got - ref).max()) <= 2e-2


def test_gate_rejects_plausible_wrong_answers():
    """The 2e-2 bf16 gate must fail an all-zero output, a dropped last block and a slot off by one."""
    wl = kvgen.make_workload("C2", variant="sharp", num_seqs=6)
    ref = oracle.run_step(wl)
    assert _bf16_gate(ref["out"], ref["out"])
    assert not _bf16_gate(np.zeros_like(ref["out"]), ref["out"])
    # last block dropped: attend over L - (L-1) % 16 - 1 tokens instead of L
    short = kvgen.dataclasses.replace(wl, context_lens=(wl.context_lens - ((wl.context_lens - 1) % 16) - 1).astype(np.int32))
    dropped = oracle.paged_attention(wl.q, ref["k_pool"], ref["v_pool"], "bf16", wl.block_tables,
                                     short.context_lens, 1 / math.sqrt(128))
    assert not _bf16_gate(dropped, ref["out"])
    # slot off by one: the scatter writes one slot further on
    kp, vp = oracle.scatter(wl.k_pool, wl.v_pool, wl.k_new, wl.v_new, ref["slots"] + 1)
    shifted = oracle.paged_attention(wl.q, kp, vp, "bf16", wl.block_tables, wl.context_lens, 1 / math.sqrt(128))
    assert not _bf16_gate(shifted, ref["out"])


def test_spec_inputs_are_weak_and_need_variants():
    """With the specified 1/sqrt(128) scaling an all-zero answer passes 2e-2: the reason for variants."""
    wl = kvgen.make_workload("C2", variant="spec", num_seqs=4)
    ref = oracle.run_step(wl)["out"]
    assert _bf16_gate(np.zeros_like(ref), ref)
    for v in ("sharp", "hot", "needle"):
        wlv = kvgen.make_workload("C2", variant=v, num_seqs=4)
        refv = oracle.run_step(wlv)["out"]
        assert not _bf16_gate(np.zeros_like(refv), refv), v


# ------------------------------------------------------------ copy-on-write --

def test_attention_through_a_copied_block_is_exact():
    """A copied block is the same data: attention through a table repointed at
    the copy equals attention through the original, bit for bit, and the pool
    differs only at the destination."""
    rng = np.random.default_rng(11)
    N, H, B, D = 12, 2, 16, 64
    kp = rng.standard_normal((N, H, B, D)).astype(np.float32)
    vp = rng.standard_normal((N, H, B, D)).astype(np.float32)
    q = rng.standard_normal((1, 4, D)).astype(np.float32)
    table = np.array([[3, 7, 1, 0]], dtype=np.int32)
    lens = np.array([53], dtype=np.int32)
    k2, v2 = oracle.copy_blocks(kp, vp, [(7, 10)])
    changed = [b for b in range(N) if not (np.array_equal(k2[b], kp[b]) and np.array_equal(v2[b], vp[b]))]
    assert changed == [10]
    moved = table.copy()
    moved[0, 1] = 10
    a = oracle.paged_attention(q, kp, vp, "f32", table, lens, 0.125)
    b = oracle.paged_attention(q, k2, v2, "f32", moved, lens, 0.125)
    assert np.array_equal(a, b)


def test_copy_blocks_skips_identity_and_out_of_range_pairs_and_copies_every_layer():
    rng = np.random.default_rng(12)
    kp = rng.standard_normal((3, 6, 2, 16, 8)).astype(np.float32)   # [layers][N][H][B][D]
    vp = rng.standard_normal((3, 6, 2, 16, 8)).astype(np.float32)
    k2, v2 = oracle.copy_blocks(kp, vp, [(2, 2), (-1, 3), (1, 6), (6, 0)])
    assert np.array_equal(k2, kp) and np.array_equal(v2, vp)
    k3, v3 = oracle.copy_blocks(kp, vp, [(4, 1), (0, 5)])
    for layer in range(3):
        assert np.array_equal(k3[layer, 1], kp[layer, 4]) and np.array_equal(v3[layer, 5], vp[layer, 0])
        assert np.array_equal(k3[layer, [0, 2, 3, 4]], kp[layer, [0, 2, 3, 4]])
