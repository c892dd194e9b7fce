"""The C-ABI library on the CPU: it loads, exports every entry point the header
declares, and its host-side logic (pool arithmetic, slot mapping, argument
checks) behaves as documented.  No kernel is launched here: every call below
either is host-only or returns an error before any HIP call.
"""
import ctypes
import json
import os
import re

import numpy as np
import pytest

import kvgen
import oracle
import paged_kv_cache_num_amd as kvp
from paged_kv_cache_num_amd import kvpool as K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = json.load(open(os.path.join(ROOT, "tests", "golden", "pages_numbers.json")))


def _declared_functions():
    names = []
    for fn in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if not fn.endswith(".h"):
            continue
        text = open(os.path.join(ROOT, "include", fn)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s+\*?([a-z_][a-z0-9_]*)\s*\(",
                            text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_expected_entry_points():
    assert set(_declared_functions()) == set(K.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(K.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(lib, name), name


def _desc(**kw):
    base = dict(num_layers=1, num_blocks=64, block_size=16, num_kv_heads=2, head_dim=64, dtype="f32")
    base.update(kw)
    return kvp.make_desc(**base)


# ---------------------------------------------------------- pool arithmetic --

def test_pool_bytes_reproduces_the_pages_per_token_figures():
    g = GOLDEN["kv_bytes_per_token_70b"]
    one_token = _desc(num_layers=g["layers"], num_blocks=1, block_size=1, num_kv_heads=g["kv_heads"],
                      head_dim=g["head_dim"], dtype="bf16")
    assert 2 * kvp.kv_pool_bytes(one_token) == g["expected_bytes"]
    r = GOLDEN["reserve_4k_70b"]
    seq = _desc(num_layers=80, num_blocks=1, block_size=r["tokens"], num_kv_heads=8, head_dim=128, dtype="bf16")
    assert 2 * kvp.kv_pool_bytes(seq) == r["expected_gib"] * 2**30
    g = GOLDEN["kv_bytes_per_token_8b"]
    tok = _desc(num_layers=g["layers"], num_blocks=1, block_size=1, num_kv_heads=g["kv_heads"],
                head_dim=g["head_dim"], dtype="bf16")
    assert 2 * kvp.kv_pool_bytes(tok) == g["expected_bytes"]
    blk = _desc(num_layers=g["layers"], num_blocks=1, block_size=g["block_size"], num_kv_heads=g["kv_heads"],
                head_dim=g["head_dim"], dtype="bf16")
    assert 2 * kvp.kv_pool_bytes(blk) == g["expected_block_bytes"]
    pool = _desc(num_layers=g["layers"], num_blocks=g["kv_budget_blocks"], block_size=16,
                 num_kv_heads=8, head_dim=128, dtype="bf16")
    assert 2 * kvp.kv_pool_bytes(pool) // g["expected_block_bytes"] * 16 == g["expected_tokens"]


def test_pool_bytes_reproduces_the_70b_capacity_printout():
    c = GOLDEN["llama70b_capacity"]
    one = _desc(num_layers=c["layers"], num_blocks=1, block_size=c["context"], num_kv_heads=c["kv_heads"],
                head_dim=c["head_dim"], dtype="bf16")
    assert 2 * kvp.kv_pool_bytes(one) / 2**30 == c["expected_gib_one_seq"]
    users = _desc(num_layers=c["layers"], num_blocks=c["users"], block_size=c["context"],
                  num_kv_heads=c["kv_heads"], head_dim=c["head_dim"], dtype="bf16")
    assert 2 * kvp.kv_pool_bytes(users) / 2**30 == c["expected_gib_users"]
    mha = _desc(num_layers=c["layers"], num_blocks=1, block_size=c["context"], num_kv_heads=c["kv_heads_mha"],
                head_dim=c["head_dim"], dtype="bf16")
    assert 2 * kvp.kv_pool_bytes(mha) / 2**30 == c["expected_gib_mha"]


def test_table_entry_counts():
    for c in GOLDEN["table_entries"]:
        # slots for the last token of the context go through entry ceil(n/B) - 1: the row must have that many
        n, B = c["tokens"], c["block_size"]
        need = c["expected_entries"]
        table = np.arange(need, dtype=np.int32)[None, :]
        s = kvp.kv_build_slot_mapping(table, B, need, [0], [n - 1], [1])
        assert s[0] == n - 1
        with pytest.raises(kvp.KVError):
            kvp.kv_build_slot_mapping(table[:, :need - 1], B, need, [0], [n - 1], [1])
        assert need * 4 == c["expected_bytes"]


def test_pool_bytes_errors():
    with pytest.raises(kvp.KVError) as e:
        kvp.kv_pool_bytes(_desc(num_blocks=0))
    assert e.value.status == K.KV_ERR_INVALID_ARGUMENT
    bad = _desc()
    bad.dtype = 7
    with pytest.raises(kvp.KVError):
        kvp.kv_pool_bytes(bad)
    with pytest.raises(kvp.KVError):
        kvp.kv_pool_bytes(_desc(num_layers=2**30, num_blocks=2**30, head_dim=2**20))


# ------------------------------------------------------------ slot mapping --

@pytest.mark.parametrize("name", ["C1", "C2", "C3", "C4", "C5"])
def test_host_slot_mapping_matches_the_oracle_bit_exactly(name):
    wl = kvgen.make_workload(name, num_seqs=None if name in ("C1", "C5") else 24)
    tables = wl.all_tables()
    got = kvp.kv_build_slot_mapping(tables, wl.block_size, wl.num_blocks, wl.write_seq,
                                    wl.write_start, wl.write_count)
    ref = oracle.slot_mapping(tables, wl.block_size, wl.num_blocks, wl.write_seq,
                              wl.write_start, wl.write_count)
    assert got.dtype == np.int64 and np.array_equal(got, ref)


def test_host_slot_mapping_errors():
    t = np.array([[3, 1]], dtype=np.int32)
    with pytest.raises(kvp.KVError) as e:
        kvp.kv_build_slot_mapping(t, 16, 4, [0], [32], [1])
    assert e.value.status == K.KV_ERR_OUT_OF_RANGE
    with pytest.raises(kvp.KVError) as e:
        kvp.kv_build_slot_mapping(np.array([[9]], dtype=np.int32), 16, 4, [0], [0], [1])
    assert e.value.status == K.KV_ERR_OUT_OF_RANGE
    with pytest.raises(kvp.KVError) as e:
        kvp.kv_build_slot_mapping(t, 16, 4, [1], [0], [1])
    assert e.value.status == K.KV_ERR_INVALID_ARGUMENT
    with pytest.raises(kvp.KVError):
        kvp.kv_build_slot_mapping(t, 16, 4, [0], [-1], [1])
    assert kvp.kv_build_slot_mapping(t, 16, 4, [0], [5], [0]).size == 0


# ------------------------------------------------------- argument checks --

FAKE_K = 0x10000000   # never dereferenced: every call below fails its host checks first
FAKE_V = 0x20000000


def _pool(**kw):
    d = _desc(**kw)
    h = ctypes.c_void_p(0)
    st = K.lib.kv_pool_create(ctypes.byref(d), FAKE_K, FAKE_V, ctypes.byref(h))
    return st, h


def test_pool_create_checks():
    st, h = _pool()
    assert st == K.KV_OK and h.value
    K.lib.kv_pool_destroy(h)
    assert _pool(block_size=32)[0] == K.KV_ERR_UNSUPPORTED
    assert _pool(head_dim=96)[0] == K.KV_ERR_UNSUPPORTED
    d = _desc()
    h = ctypes.c_void_p(0)
    assert K.lib.kv_pool_create(ctypes.byref(d), FAKE_K + 8, FAKE_V, ctypes.byref(h)) == K.KV_ERR_INVALID_ARGUMENT
    assert K.lib.kv_pool_create(ctypes.byref(d), None, FAKE_V, ctypes.byref(h)) == K.KV_ERR_INVALID_ARGUMENT
    assert b"NULL" in K.lib.kv_last_error_message()
    assert K.lib.kv_pool_destroy(None) == K.KV_OK


def _decode(h, **kw):
    a = dict(layer=0, out=0x30000000, q=0x40000000, tables=0x50000000, mb=16, lens=0x60000000, S=4, Hq=8,
             scale=0.125, max_ctx=200, part=0, ws=None, ws_bytes=0)
    a.update(kw)
    return K.lib.paged_attention_decode(h, a["layer"], a["out"], a["q"], a["tables"], a["mb"], a["lens"], a["S"],
                                        a["Hq"], a["scale"], a["max_ctx"], a["part"], a["ws"], a["ws_bytes"], None)


def test_decode_argument_checks_return_before_any_launch():
    st, h = _pool()
    assert st == K.KV_OK
    E = K
    assert _decode(None) == E.KV_ERR_INVALID_ARGUMENT
    assert _decode(h, layer=1) == E.KV_ERR_INVALID_ARGUMENT
    assert _decode(h, Hq=7) == E.KV_ERR_INVALID_ARGUMENT          # not a multiple of 2 KV heads
    assert _decode(h, Hq=6) == E.KV_ERR_UNSUPPORTED               # group of 3
    assert _decode(h, Hq=32) == E.KV_ERR_UNSUPPORTED              # group of 16
    assert _decode(h, part=40) == E.KV_ERR_INVALID_ARGUMENT       # not a multiple of B
    assert _decode(h, max_ctx=16 * 16 + 1) == E.KV_ERR_INVALID_ARGUMENT
    assert _decode(h, scale=float("nan")) == E.KV_ERR_INVALID_ARGUMENT
    assert _decode(h, scale=0.0) == E.KV_ERR_INVALID_ARGUMENT
    assert _decode(h, scale=-0.5) == E.KV_ERR_INVALID_ARGUMENT
    assert _decode(h, out=0x30000008) == E.KV_ERR_INVALID_ARGUMENT
    assert _decode(h, q=None) == E.KV_ERR_INVALID_ARGUMENT
    assert _decode(h, part=64) == E.KV_ERR_WORKSPACE_TOO_SMALL
    need = ctypes.c_uint64(0)
    assert K.lib.paged_attention_workspace_bytes(h, 4, 8, 200, 64, ctypes.byref(need)) == E.KV_OK
    assert _decode(h, part=64, ws=0x70000000, ws_bytes=need.value - 1) == E.KV_ERR_WORKSPACE_TOO_SMALL
    assert _decode(h, S=0) == E.KV_OK                              # nothing to do, nothing launched
    K.lib.kv_pool_destroy(h)


def test_decode_append_argument_checks_return_before_any_launch():
    st, h = _pool()
    L = K.lib
    args = [0, 0x30000000, 0x40000000, 0x70000000, 0x78000000, 0x50000000, 16, 0x60000000, 4, 8, 0.125, 200, 0,
            None, 0, None]
    def call(**kw):
        a = list(args)
        for k, v in kw.items():
            a[{"k": 3, "v": 4, "S": 8, "Hq": 9, "scale": 10}[k]] = v
        return L.paged_attention_decode_append(h, *a)
    assert L.paged_attention_decode_append(None, *args) == K.KV_ERR_INVALID_ARGUMENT
    assert call(k=None) == K.KV_ERR_INVALID_ARGUMENT
    assert call(v=None) == K.KV_ERR_INVALID_ARGUMENT
    assert call(k=0x70000008) == K.KV_ERR_INVALID_ARGUMENT        # misaligned new row
    assert call(Hq=6) == K.KV_ERR_UNSUPPORTED                      # group of 3, as for the plain call
    assert call(scale=0.0) == K.KV_ERR_INVALID_ARGUMENT
    assert call(S=0, k=None, v=None) == K.KV_OK                    # nothing to do, nothing launched
    K.lib.kv_pool_destroy(h)


def test_block_size_support():
    """B in {8, 16, 32, 64, 128} for bf16 pools with head_dim 128; B = 16 for the others."""
    import ctypes
    for B, dt, d, want in [(8, "bf16", 128, K.KV_OK), (128, "bf16", 128, K.KV_OK),
                           (24, "bf16", 128, K.KV_ERR_UNSUPPORTED), (256, "bf16", 128, K.KV_ERR_UNSUPPORTED),
                           (32, "f32", 64, K.KV_ERR_UNSUPPORTED), (32, "bf16", 64, K.KV_ERR_UNSUPPORTED),
                           (16, "f32", 64, K.KV_OK)]:
        desc = K.make_desc(1, 8, B, 2, d, dt)
        h = ctypes.c_void_p()
        st = K.lib.kv_pool_create(ctypes.byref(desc), 0x10000, 0x20000, ctypes.byref(h))
        assert st == want, (B, dt, d, st)
        if st == K.KV_OK:
            K.lib.kv_pool_destroy(h)


def test_workspace_size_formula():
    st, h = _pool(head_dim=128, num_kv_heads=8, dtype="bf16")
    out = ctypes.c_uint64(0)
    # partitions: (m, l) pairs padded to 256 bytes, then D fp32 per (seq, head, partition)
    assert K.lib.paged_attention_workspace_bytes(h, 8, 32, 131072, 512, ctypes.byref(out)) == K.KV_OK
    parts = 131072 // 512
    entries = 8 * 32 * parts
    assert out.value == -(-entries * 8 // 256) * 256 + entries * 128 * 4
    # one partition covering the longest context: no workspace
    assert K.lib.paged_attention_workspace_bytes(h, 8, 32, 4096, 4096, ctypes.byref(out)) == K.KV_OK
    assert out.value == 0
    # balanced split: tile prefix sums, then two partial states (4 heads x 128 fp32 + 8 fp32) per worker
    assert K.lib.paged_attention_workspace_bytes(h, 64, 32, 4096, 0, ctypes.byref(out)) == K.KV_OK
    prefix = -(-(64 + 1) * 8 // 256) * 256
    workers, rem = divmod(out.value - prefix, 2 * (4 * 128 + 8) * 4)
    assert rem == 0 and workers >= 1
    K.lib.kv_pool_destroy(h)
    # fp32 pools walk each context in one workgroup: no workspace
    st, h = _pool(head_dim=64, num_kv_heads=2, dtype="f32")
    assert K.lib.paged_attention_workspace_bytes(h, 4, 8, 200, 0, ctypes.byref(out)) == K.KV_OK
    assert out.value == 0
    K.lib.kv_pool_destroy(h)


def test_table_walk_probe_argument_checks():
    L = K.lib
    # null pointers, bad sizes and a context longer than the table rows fail before any launch
    assert L.kv_probe_table_walk(None, 4, 0x1000, 2, 8, 64, 0, 0x2000, 4096, None) == K.KV_ERR_INVALID_ARGUMENT
    assert L.kv_probe_table_walk(0x1000, 4, None, 2, 8, 64, 0, 0x2000, 4096, None) == K.KV_ERR_INVALID_ARGUMENT
    assert L.kv_probe_table_walk(0x1000, 4, 0x1000, 2, 8, 64, 0, None, 4096, None) == K.KV_ERR_INVALID_ARGUMENT
    assert L.kv_probe_table_walk(0x1000, 4, 0x1000, -1, 8, 64, 0, 0x2000, 4096, None) == K.KV_ERR_INVALID_ARGUMENT
    assert L.kv_probe_table_walk(0x1000, 4, 0x1000, 2, 0, 64, 0, 0x2000, 4096, None) == K.KV_ERR_INVALID_ARGUMENT
    assert L.kv_probe_table_walk(0x1000, 4, 0x1000, 2, 8, 65, 0, 0x2000, 4096, None) == K.KV_ERR_INVALID_ARGUMENT
    assert L.kv_probe_table_walk(0x1000, 4, 0x1000, 2, 8, 64, 0, 0x2002, 4096, None) == K.KV_ERR_INVALID_ARGUMENT


def test_scatter_argument_checks():
    st, h = _pool()
    L = K.lib
    assert L.reshape_and_cache(None, 0, 0x1000, 0x2000, 0x3000, 4, None) == K.KV_ERR_INVALID_ARGUMENT
    assert L.reshape_and_cache(h, 3, 0x1000, 0x2000, 0x3000, 4, None) == K.KV_ERR_INVALID_ARGUMENT
    assert L.reshape_and_cache(h, 0, 0x1008, 0x2000, 0x3000, 4, None) == K.KV_ERR_INVALID_ARGUMENT
    assert L.reshape_and_cache(h, 0, 0x1000, 0x2000, 0x3004, 4, None) == K.KV_ERR_INVALID_ARGUMENT
    assert L.reshape_and_cache(h, 0, 0x1000, 0x2000, None, 4, None) == K.KV_ERR_INVALID_ARGUMENT
    assert L.reshape_and_cache(h, 0, 0x1000, 0x2000, 0x3000, -1, None) == K.KV_ERR_INVALID_ARGUMENT
    assert L.reshape_and_cache(h, 0, 0x1000, 0x2000, 0x3000, 0, None) == K.KV_OK
    K.lib.kv_pool_destroy(h)
    # the scatter numbers a token's chunks in 32 bits: at most 2^20 KV heads
    st, big = _pool(num_kv_heads=(1 << 20) + 1, num_blocks=1)
    assert st == K.KV_OK
    assert L.reshape_and_cache(big, 0, 0x1000, 0x2000, 0x3000, 4, None) == K.KV_ERR_UNSUPPORTED
    K.lib.kv_pool_destroy(big)


def test_status_strings():
    for code, name in [(0, "KV_OK"), (-1, "KV_ERR_INVALID_ARGUMENT"), (-2, "KV_ERR_UNSUPPORTED"),
                       (-3, "KV_ERR_WORKSPACE_TOO_SMALL"), (-4, "KV_ERR_HIP"), (-5, "KV_ERR_OUT_OF_RANGE")]:
        assert K.lib.kv_status_string(code).decode() == name
    assert K.lib.kv_status_string(42).decode() == "KV_ERR_UNKNOWN"


# ------------------------------------------------------------------ FP8 pools --

def _fp8_pool(**kw):
    d = _desc(**dict(dict(head_dim=128, num_kv_heads=2, dtype="fp8"), **kw))
    h = ctypes.c_void_p(0)
    st = K.lib.kv_pool_create_fp8(ctypes.byref(d), 0x10000, 0x20000, 0x30000, 0x40000, ctypes.byref(h))
    return st, h


def test_fp8_pool_sizes():
    """Codes are one byte per element; scales one fp32 per (layer, block, KV head) and tensor."""
    d = _desc(num_layers=3, num_blocks=10, block_size=16, num_kv_heads=8, head_dim=128, dtype="fp8")
    assert kvp.kv_pool_bytes(d) == 3 * 10 * 16 * 8 * 128
    assert K.kv_pool_scale_bytes(d) == 3 * 10 * 8 * 4
    # the bf16 pool of the same shape is twice the code bytes and has no scales
    d16 = _desc(num_layers=3, num_blocks=10, block_size=16, num_kv_heads=8, head_dim=128, dtype="bf16")
    assert kvp.kv_pool_bytes(d16) == 2 * kvp.kv_pool_bytes(d)
    assert K.kv_pool_scale_bytes(d16) == 0


def test_fp8_pool_create_checks():
    st, h = _fp8_pool()
    assert st == K.KV_OK and h.value
    K.lib.kv_pool_destroy(h)
    # an FP8 descriptor needs the FP8 entry point, and that entry point an FP8 descriptor
    d = _desc(head_dim=128, dtype="fp8")
    h = ctypes.c_void_p(0)
    assert K.lib.kv_pool_create(ctypes.byref(d), 0x10000, 0x20000, ctypes.byref(h)) == K.KV_ERR_INVALID_ARGUMENT
    d16 = _desc(head_dim=128, dtype="bf16")
    assert K.lib.kv_pool_create_fp8(ctypes.byref(d16), 0x10000, 0x20000, 0x30000, 0x40000,
                                    ctypes.byref(h)) == K.KV_ERR_INVALID_ARGUMENT
    # scales: non-null, 4-byte aligned
    assert K.lib.kv_pool_create_fp8(ctypes.byref(d), 0x10000, 0x20000, None, 0x40000,
                                    ctypes.byref(h)) == K.KV_ERR_INVALID_ARGUMENT
    assert K.lib.kv_pool_create_fp8(ctypes.byref(d), 0x10000, 0x20000, 0x30002, 0x40000,
                                    ctypes.byref(h)) == K.KV_ERR_INVALID_ARGUMENT
    # built for head_dim 128 and the block sizes of the bf16 / head_dim-128 pools
    assert _fp8_pool(head_dim=64)[0] == K.KV_ERR_UNSUPPORTED
    for B in (8, 16, 32, 64, 128):
        st, h = _fp8_pool(block_size=B)
        assert st == K.KV_OK, B
        K.lib.kv_pool_destroy(h)
    for B in (4, 24, 256):
        assert _fp8_pool(block_size=B)[0] == K.KV_ERR_UNSUPPORTED, B


def test_fp8_decode_argument_checks():
    st, h = _fp8_pool()
    assert st == K.KV_OK
    assert _decode(h, Hq=6) == K.KV_ERR_UNSUPPORTED                # group of 3
    assert _decode(h, part=24) == K.KV_ERR_INVALID_ARGUMENT        # not a multiple of 16
    assert _decode(h, part=64) == K.KV_ERR_WORKSPACE_TOO_SMALL
    # the balanced split is used for FP8 pools too: a workspace is needed with partition_size 0
    need = ctypes.c_uint64(0)
    assert K.lib.paged_attention_workspace_bytes(h, 4, 8, 200, 0, ctypes.byref(need)) == K.KV_OK
    assert need.value > 0
    assert _decode(h) == K.KV_ERR_WORKSPACE_TOO_SMALL
    assert _decode(h, S=0) == K.KV_OK
    K.lib.kv_pool_destroy(h)


def test_fp8_probe_argument_checks():
    L = K.lib
    assert L.kv_probe_e4m3_to_bf16(None, 0x2000, 4, None) == K.KV_ERR_INVALID_ARGUMENT
    assert L.kv_probe_e4m3_to_bf16(0x1000, 0x2001, 4, None) == K.KV_ERR_INVALID_ARGUMENT
    assert L.kv_probe_e4m3_to_bf16(0x1000, 0x2000, -1, None) == K.KV_ERR_INVALID_ARGUMENT
    assert L.kv_probe_e4m3_to_bf16(None, None, 0, None) == K.KV_OK
    assert L.kv_probe_f32_to_e4m3(0x1002, 0x2000, 4, None) == K.KV_ERR_INVALID_ARGUMENT
    assert L.kv_probe_f32_to_e4m3(None, None, 0, None) == K.KV_OK


# -------------------------------------------------------------------- swap --

def test_swap_bytes_reproduce_the_pages_figures():
    """A 4K-token 70B-class sequence swaps 1.25 GiB each way; a block of the
    8B-class pool is 2 MiB; at 25 GB/s a trip takes about 50 ms."""
    g = GOLDEN["swap_4k_70b"]
    d = _desc(num_layers=g["layers"], num_blocks=300, block_size=g["block_size"], num_kv_heads=g["kv_heads"],
              head_dim=g["head_dim"], dtype="bf16")
    h = ctypes.c_void_p(0)
    assert K.lib.kv_pool_create(ctypes.byref(d), 0x10000, 0x20000, ctypes.byref(h)) == K.KV_OK
    out = ctypes.c_uint64(0)
    assert K.lib.kv_swap_bytes(h, g["tokens"] // g["block_size"], ctypes.byref(out)) == K.KV_OK
    assert out.value == g["expected_gib_each_way"] * 2**30
    seconds = out.value / (g["link_gb_per_s"] * 1e9)
    assert abs(seconds * 1e3 - g["expected_ms_each_way"]) / g["expected_ms_each_way"] < 0.1
    K.lib.kv_pool_destroy(h)
    b = GOLDEN["kv_bytes_per_token_8b"]
    d8 = _desc(num_layers=b["layers"], num_blocks=10, block_size=b["block_size"], num_kv_heads=b["kv_heads"],
               head_dim=b["head_dim"], dtype="bf16")
    assert K.lib.kv_pool_create(ctypes.byref(d8), 0x10000, 0x20000, ctypes.byref(h)) == K.KV_OK
    assert K.lib.kv_swap_bytes(h, 1, ctypes.byref(out)) == K.KV_OK
    assert out.value == b["expected_block_bytes"]
    K.lib.kv_pool_destroy(h)


def test_swap_bytes_match_the_oracle_record_for_fp8_pools():
    for layers, heads in [(1, 1), (3, 8), (2, 3)]:
        st, h = _fp8_pool(num_layers=layers, num_kv_heads=heads)
        assert st == K.KV_OK
        out = ctypes.c_uint64(0)
        assert K.lib.kv_swap_bytes(h, 5, ctypes.byref(out)) == K.KV_OK
        assert out.value == 5 * oracle.swap_record_bytes(layers, heads * 16 * 128, heads, fp8=True)
        assert out.value % 16 == 0
        K.lib.kv_pool_destroy(h)


def test_swap_argument_checks_return_before_any_launch():
    st, h = _pool(head_dim=128, dtype="bf16")
    L = K.lib
    need = ctypes.c_uint64(0)
    assert L.kv_swap_bytes(h, 4, ctypes.byref(need)) == K.KV_OK
    buf = np.zeros(need.value + 16, dtype=np.uint8)
    host = (buf.ctypes.data + 15) // 16 * 16
    for fn in (L.kv_swap_out, L.kv_swap_in):
        assert fn(None, 0x1000, 4, host, need.value, None) == K.KV_ERR_INVALID_ARGUMENT
        assert fn(h, 0x1000, -1, host, need.value, None) == K.KV_ERR_INVALID_ARGUMENT
        assert fn(h, None, 4, host, need.value, None) == K.KV_ERR_INVALID_ARGUMENT
        assert fn(h, 0x1002, 4, host, need.value, None) == K.KV_ERR_INVALID_ARGUMENT
        assert fn(h, 0x1000, 4, host + 8, need.value, None) == K.KV_ERR_INVALID_ARGUMENT
        assert fn(h, 0x1000, 4, host, need.value - 16, None) == K.KV_ERR_INVALID_ARGUMENT
        # ordinary (pageable) host memory is refused: the kernels need a pinned, mapped buffer
        assert fn(h, 0x1000, 4, host, need.value, None) == K.KV_ERR_INVALID_ARGUMENT
        assert b"pinned" in L.kv_last_error_message() or b"mapping" in L.kv_last_error_message()
        assert fn(h, None, 0, None, 0, None) == K.KV_OK
    K.lib.kv_pool_destroy(h)


def test_bench_refuses_more_than_one_gpu():
    """bench.py runs the hot path on one GPU; --gpus above 1 exits with a message."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def _shared(h, **kw):
    a = dict(layer=0, out=0x30000000, q=0x40000000, tables=0x50000000, mb=256, lens=0x60000000, S=4, Hq=32,
             scale=0.125, max_ctx=4096, shared=128, ws=None, ws_bytes=0)
    a.update(kw)
    return K.lib.paged_attention_decode_shared(h, a["layer"], a["out"], a["q"], a["tables"], a["mb"], a["lens"],
                                               a["S"], a["Hq"], a["scale"], a["max_ctx"], a["shared"], a["ws"],
                                               a["ws_bytes"], None)


def _shared_ws(h, S=4, Hq=32, max_ctx=4096, mb=256, shared=128):
    out = ctypes.c_uint64(0)
    st = K.lib.paged_attention_shared_workspace_bytes(h, S, Hq, max_ctx, mb, shared, ctypes.byref(out))
    return st, int(out.value)


def test_shared_prefix_argument_checks_return_before_any_launch():
    # a bf16 pool with head_dim 128 and block size 16, as the shared-prefix kernels need
    st, h = _pool(num_kv_heads=8, head_dim=128, dtype="bf16", num_blocks=1024)
    assert st == K.KV_OK
    assert _shared(None) == K.KV_ERR_INVALID_ARGUMENT
    assert _shared(h, shared=-1) == K.KV_ERR_INVALID_ARGUMENT
    assert _shared(h, shared=257) == K.KV_ERR_INVALID_ARGUMENT           # past max_blocks_per_seq
    assert _shared(h, shared=129, max_ctx=2063) == K.KV_ERR_INVALID_ARGUMENT   # past max_context_len / B
    assert _shared(h, Hq=24) == K.KV_ERR_UNSUPPORTED                     # group of 3
    assert _shared(h, S=0) == K.KV_OK                                    # nothing to do
    st, need = _shared_ws(h)
    assert st == K.KV_OK and need > 0
    assert _shared(h, ws=0x70000000, ws_bytes=need - 1) == K.KV_ERR_WORKSPACE_TOO_SMALL
    assert _shared(h, ws=0x70000008, ws_bytes=need) == K.KV_ERR_INVALID_ARGUMENT   # misaligned
    # shared_blocks 0: the plain call's workspace
    st, plain = _shared_ws(h, shared=0)
    want = ctypes.c_uint64(0)
    assert K.lib.paged_attention_workspace_bytes(h, 4, 32, 4096, 0, ctypes.byref(want)) == K.KV_OK
    assert st == K.KV_OK and plain == want.value
    # the prefix states come on top of the balanced split's workspace
    assert need > plain
    assert _shared_ws(h, shared=-1)[0] == K.KV_ERR_INVALID_ARGUMENT
    K.lib.kv_pool_destroy(h)
    # other pools: unsupported
    for kw in (dict(), dict(num_kv_heads=8, head_dim=64, dtype="bf16")):
        st, h = _pool(**kw)
        assert st == K.KV_OK
        assert _shared(h, Hq=8 * (kw.get("num_kv_heads", 2) // 2)) == K.KV_ERR_UNSUPPORTED
        assert _shared_ws(h, Hq=8 * (kw.get("num_kv_heads", 2) // 2))[0] == K.KV_ERR_UNSUPPORTED
        K.lib.kv_pool_destroy(h)
    # bf16 / head_dim 128 at other block sizes: supported; the prefix states come on top of
    # the plain workspace once the prefix holds a whole 16-token tile (one 8-token block does not)
    for B, shared, extra in ((32, 4, True), (128, 2, True), (8, 2, True), (8, 1, False)):
        st, h = _pool(num_kv_heads=8, head_dim=128, dtype="bf16", block_size=B)
        assert st == K.KV_OK
        st, need = _shared_ws(h, Hq=32, shared=shared)
        assert st == K.KV_OK
        plain = ctypes.c_uint64(0)
        assert K.lib.paged_attention_workspace_bytes(h, 4, 32, 4096, 0, ctypes.byref(plain)) == K.KV_OK
        assert (need > plain.value) == extra, (B, shared)
        K.lib.kv_pool_destroy(h)


def test_noalloc_decode_checks_return_before_any_launch():
    """paged_attention_decode_noalloc: the same argument checks as the plain
    call, and a call needing more than the static array's bytes is refused
    with a clear error before any device work."""
    st, h = _pool(head_dim=128, num_kv_heads=8, dtype="bf16", num_blocks=64)
    L = K.lib

    def call(**kw):
        a = dict(layer=0, out=0x30000000, q=0x40000000, tables=0x50000000, mb=8192, lens=0x60000000, S=4, Hq=32,
                 scale=0.125, max_ctx=200, part=0)
        a.update(kw)
        return L.paged_attention_decode_noalloc(h, a["layer"], a["out"], a["q"], a["tables"], a["mb"], a["lens"],
                                                a["S"], a["Hq"], a["scale"], a["max_ctx"], a["part"], None)
    assert L.paged_attention_decode_noalloc(None, 0, 0x30000000, 0x40000000, 0x50000000, 16, 0x60000000, 4, 32,
                                            0.125, 200, 0, None) == K.KV_ERR_INVALID_ARGUMENT
    assert call(layer=1) == K.KV_ERR_INVALID_ARGUMENT
    assert call(Hq=24) == K.KV_ERR_UNSUPPORTED                     # group of 3
    assert call(scale=0.0) == K.KV_ERR_INVALID_ARGUMENT
    assert call(part=40) == K.KV_ERR_INVALID_ARGUMENT
    # 1024 sequences of 128K tokens in 16-token partitions: far more workspace than the array holds
    need = ctypes.c_uint64(0)
    assert L.paged_attention_workspace_bytes(h, 1024, 32, 131072, 16, ctypes.byref(need)) == K.KV_OK
    assert need.value > K.KV_NOALLOC_SCRATCH_BYTES
    assert call(S=1024, max_ctx=131072, part=16) == K.KV_ERR_WORKSPACE_TOO_SMALL
    msg = L.kv_last_error_message().decode()
    assert "static array" in msg and str(K.KV_NOALLOC_SCRATCH_BYTES) in msg, msg
    assert call(S=0) == K.KV_OK                                    # nothing to do, nothing launched
    L.kv_pool_destroy(h)


def test_decode_step_row_checks_return_before_any_launch():
    """paged_attention_decode_step: the other rows' arguments are checked
    (count, NULL pointers, alignment) before any device work, as are the
    decode arguments; no rows and no sequences is a no-op."""
    st, h = _pool(head_dim=128, num_kv_heads=8, dtype="bf16", num_blocks=64)
    L = K.lib

    def call(**kw):
        a = dict(layer=0, out=0x30000000, q=0x40000000, kn=0x70000000, vn=0x71000000, tables=0x50000000, mb=16,
                 lens=0x60000000, S=4, Hq=32, scale=0.125, max_ctx=200, part=0, kr=0x72000000, vr=0x73000000,
                 slots=0x74000000, R=2048, ws=None, wsb=0)
        a.update(kw)
        return L.paged_attention_decode_step(h, a["layer"], a["out"], a["q"], a["kn"], a["vn"], a["tables"], a["mb"],
                                             a["lens"], a["S"], a["Hq"], a["scale"], a["max_ctx"], a["part"],
                                             a["kr"], a["vr"], a["slots"], a["R"], a["ws"], a["wsb"], None)
    assert call(R=-1) == K.KV_ERR_INVALID_ARGUMENT
    assert call(kr=None) == K.KV_ERR_INVALID_ARGUMENT
    assert call(slots=None) == K.KV_ERR_INVALID_ARGUMENT
    assert call(vr=0x73000008) == K.KV_ERR_INVALID_ARGUMENT         # not 16-byte aligned
    assert call(slots=0x74000004) == K.KV_ERR_INVALID_ARGUMENT      # not 8-byte aligned
    assert call(kn=None) == K.KV_ERR_INVALID_ARGUMENT
    assert call(layer=1) == K.KV_ERR_INVALID_ARGUMENT
    assert call(Hq=24) == K.KV_ERR_UNSUPPORTED
    assert call(part=40) == K.KV_ERR_INVALID_ARGUMENT
    assert call(S=0, R=0) == K.KV_OK                                 # nothing to do, nothing launched
    L.kv_pool_destroy(h)
