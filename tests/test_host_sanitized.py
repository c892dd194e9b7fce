"""Host code built with g++ under the address and undefined-behaviour
sanitizers (CPU only).

* tests/host/split_check.cpp: the integer arithmetic the balanced decode
  shares with its fix-up (slice boundaries, the worker holding a split
  position, the positions each (sequence, KV head) walk takes) and the
  table-entry arithmetic of the tile walks, checked on many random batches
  (every tile walked once, the fix-up finds exactly the records left)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_num_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _build_and_run(tmp_path, sources, out_name, extra=(), args=()):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    exe = str(tmp_path / out_name)
    cmd = [gxx, "-std=c++17", "-O1", "-g", *SAN, "-I", CSRC, *extra, *sources, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe, *args], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    return r.stdout


def test_split_and_table_index_arithmetic_sanitized(tmp_path):
    out = _build_and_run(tmp_path, [os.path.join(ROOT, "tests", "host", "split_check.cpp")], "split_check")
    assert out.strip().endswith("ok")
