"""MI355X-native paged KV-cache hot path: slot-mapping scatter and paged decode
attention as hand-written HIP kernels for gfx950, behind the C ABI declared in
include/kvpool.h.  This package is the binding (argument marshalling) plus a
small helper that keeps one step's device buffers together.

The HIP library is loaded on first use of any name below; if it is not built,
that first use raises ImportError (there is no CPU fallback).  Importing the
``build`` submodule does not load it.
"""
import importlib

_FROM_KVPOOL = ("KV_BF16", "KV_F32", "KV_FP8_E4M3", "KVError", "KVPool", "kv_build_slot_mapping", "kv_pool_bytes",
                "kv_pool_scale_bytes", "probe_e4m3_to_bf16", "probe_f32_to_e4m3",
                "make_desc", "lib", "LIB_PATH", "EXPORTED", "probe_copy", "probe_read", "probe_table_walk")

__all__ = list(_FROM_KVPOOL) + ["DecodeStep"]


def __getattr__(name):
    if name in _FROM_KVPOOL:
        return getattr(importlib.import_module(".kvpool", __name__), name)
    if name == "DecodeStep":
        return importlib.import_module(".step", __name__).DecodeStep
    raise AttributeError(name)
