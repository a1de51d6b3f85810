"""The host layer of libssa (argument validation, geometry, workspace sizes,
error strings) under AddressSanitizer: the C-ABI and binding tests run in a
child process against the host-ASan build of the same sources
(build.build_asan), with the sanitizer runtime preloaded.  No GPU calls."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

import pytest

from block_sparse_attention_kv_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _stale() -> bool:
    if not os.path.exists(build.ASAN_LIB):
        return True
    t = os.path.getmtime(build.ASAN_LIB)
    srcs = glob.glob(os.path.join(build.CSRC, "*")) + glob.glob(os.path.join(ROOT, "include", "*.h"))
    return any(os.path.getmtime(s) > t for s in srcs)


def test_host_layer_under_asan():
    rt = build.asan_runtime()
    if rt is None:
        pytest.skip("no AddressSanitizer runtime in this toolchain")
    if _stale():
        build.build_asan()
    undefined = subprocess.run(["nm", "-D", "--undefined-only", build.ASAN_LIB], capture_output=True, text=True).stdout
    assert "__asan_report" in undefined, "the library is not instrumented"
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               SSA_LIBRARY=build.ASAN_LIB)
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_abi_cpu.py", "tests/test_binding_validation.py",
                        "-q", "-m", "not gpu", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, out
    assert "AddressSanitizer" not in r.stderr, out
    assert " passed" in r.stdout, out
