"""Shared helpers for the GPU parity tests (HIP path vs CPU oracle)."""
from __future__ import annotations

import functools
import math
import sys

import numpy as np

import kvgen
import oracle

TOL = {"f32": 1e-4, "bf16": 2e-2}


def to_f64(a, dtype):
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    return kvgen.bf16_bits_to_f32(a).astype(np.float64)


def say(*args):
    print(*args, flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=8)
def workload(name, variant="spec", poison=True, num_seqs=None):
    return kvgen.make_workload(name, variant=variant, poison=poison, num_seqs=num_seqs)


@functools.lru_cache(maxsize=8)
def reference(name, variant="spec", poison=True, num_seqs=None):
    return oracle.run_step(workload(name, variant, poison, num_seqs))


def run_gpu(wl, **kw):
    import torch
    from paged_kv_cache_num_amd import DecodeStep
    step = DecodeStep.from_workload(wl, **kw)
    step.run()
    torch.cuda.synchronize()
    return step


def max_err(gpu_out, ref_out, dtype):
    g = to_f64(gpu_out, dtype)
    assert np.isfinite(g).all(), "non-finite output"
    return float(np.abs(g - ref_out).max()) if g.size else 0.0


def check_step(step, wl, ref, *, check_pool=True, label=""):
    """Slots and pools bit-exact, attention within the dtype's tolerance."""
    assert np.array_equal(step.slots_host, ref["slots"]), f"{label}: slot mapping differs"
    if check_pool:
        kp, vp = step.pool_host()
        assert kp.tobytes() == ref["k_pool"].tobytes(), f"{label}: K pool differs after the scatter"
        assert vp.tobytes() == ref["v_pool"].tobytes(), f"{label}: V pool differs after the scatter"
    err = max_err(step.out_host(), ref["out"], wl.dtype)
    say(f"  {label}: max |gpu - oracle| = {err:.3e} (tol {TOL[wl.dtype]:.0e})")
    assert err <= TOL[wl.dtype], f"{label}: error {err} above {TOL[wl.dtype]}"
    return err
