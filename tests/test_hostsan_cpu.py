"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

The library is built a second time with the host code instrumented (the device code is
built as usual) and the CPU tests of the C ABI run against it in a child process with
the sanitizer runtime preloaded: argument validation, overlap checks, size limits and
the int32 narrowing of the plan (tests/test_abi_cpu.py), and the planner's tile and
split decisions on the benchmark, test and seeded random sets (tests/test_plan_cpu.py).
Any sanitizer report aborts the child, and the test fails.
"""
import os
import subprocess
import sys

import pytest

from matrix_orthogonalising_optimizer_02_amd import build as BUILD

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import ctypes, os, sys
sys.path.insert(0, {root!r})
from matrix_orthogonalising_optimizer_02_amd import binding as B
lib = B.load_library()
assert lib._name == {lib!r}, lib._name
ctypes.CDLL(None).__asan_init  # the sanitizer runtime is live in this process
import pytest
sys.exit(pytest.main(["-x", "-q", "-p", "no:cacheprovider", "tests/test_abi_cpu.py", "tests/test_plan_cpu.py"]))
"""


def _stale(lib):
    if not os.path.exists(lib):
        return True
    t = os.path.getmtime(lib)
    srcs = [os.path.join(BUILD.CSRC, f) for f in os.listdir(BUILD.CSRC)] + [os.path.join(ROOT, "include", "muon_rocm.h")]
    return any(os.path.getmtime(p) > t for p in srcs)


@pytest.fixture(scope="module")
def sanitized_lib():
    lib = BUILD.SANITIZED_LIB_PATH
    if _stale(lib):
        BUILD.build(out=lib, host_sanitize=True)
    return lib


def test_abi_cpu_tests_under_host_sanitizers(sanitized_lib):
    try:
        runtime = BUILD.sanitizer_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    env = dict(os.environ, MUON_ROCM_LIBRARY=sanitized_lib, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([sys.executable, "-c", CHILD.format(root=ROOT, lib=sanitized_lib)], cwd=ROOT, env=env,
                         stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=600)
    out = res.stdout
    assert res.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out, out[-2000:]
