"""The host side of the library under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

lib/libfd_sanitized.so is the same library with its host code instrumented
(`python -m decode_attention_06_amd.build --sanitized`; __graft_entry__.build()
makes it too).  The ABI tests (argument checks, planner, workspace sizing,
testing and validation switches, the allocation-free entry point's checks)
run in a child process with the ASan runtime preloaded and every report
fatal; the instrumented library cannot even load without that runtime.
"""

import os
import subprocess
import sys

import pytest

from decode_attention_06_amd import build as fdbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_tests_pass_under_asan_and_ubsan():
    runtime = fdbuild.sanitizer_runtime()
    if runtime is None:
        pytest.skip("no AddressSanitizer runtime next to hipcc")
    lib = fdbuild.SANITIZED_LIB_PATH
    srcs = [os.path.join(fdbuild.CSRC, s) for s in fdbuild.SOURCES]
    if not os.path.exists(lib) or os.path.getmtime(lib) < max(os.path.getmtime(s) for s in srcs):
        fdbuild.build(sanitized=True)
    env = dict(os.environ, LD_PRELOAD=runtime, FD_LIBRARY_PATH=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q", "-x",
                        "-p", "no:cacheprovider", "-m", "not gpu"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
