"""Host code built with g++ under the address and undefined-behaviour
sanitizers (CPU only).

* tests/host/split_check.cpp: the integer arithmetic the balanced decode
  shares with its fix-up (slice boundaries, the worker holding a split
  position, the positions each (sequence, KV head) walk takes) and the
  table-entry arithmetic of the tile walks, checked on many random batches
  (every tile walked once, the fix-up finds exactly the records left).
* tests/host/host_check.cpp: the C-ABI layer's host-only checks
  (paged_kv_cache_num_amd/csrc/host_logic.hpp: pool and scale sizes, the
  descriptor, the slot mapping and its error returns), as the release build
  compiles them and as the KV_DEBUG build does (which also refuses two writes
  to one slot in a call).
* tests/host/oracle_check.c: the CPU oracle (oracle/oracle.c) with gcc, on
  cases with closed forms and its error returns."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_num_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


INCLUDE = os.path.join(ROOT, "include")


def _build_and_run(tmp_path, sources, out_name, extra=(), args=(), compiler="g++", std="-std=c++17", libs=()):
    cc = shutil.which(compiler)
    if cc is None:
        pytest.skip(f"{compiler} not found")
    exe = str(tmp_path / out_name)
    cmd = [cc, std, "-O1", "-g", *SAN, "-I", CSRC, "-I", INCLUDE, *extra, *sources, "-o", exe, *libs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe, *args], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    return r.stdout


def test_split_and_table_index_arithmetic_sanitized(tmp_path):
    out = _build_and_run(tmp_path, [os.path.join(ROOT, "tests", "host", "split_check.cpp")], "split_check")
    assert out.strip().endswith("ok")


@pytest.mark.parametrize("debug", [0, 1])
def test_abi_host_checks_sanitized(tmp_path, debug):
    out = _build_and_run(tmp_path, [os.path.join(ROOT, "tests", "host", "host_check.cpp")], f"host_check{debug}",
                         extra=[f"-DCHECK_DEBUG={debug}"])
    assert out.strip().endswith("ok")


def test_oracle_sanitized(tmp_path):
    out = _build_and_run(tmp_path, [os.path.join(ROOT, "oracle", "oracle.c"),
                                    os.path.join(ROOT, "tests", "host", "oracle_check.c")],
                         "oracle_check", extra=["-pthread"], compiler="gcc", std="-std=c11", libs=["-lm"])
    assert out.strip().endswith("ok")
