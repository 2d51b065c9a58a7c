"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds the host-sanitized library (``build(sanitize=True)``: -fsanitize=address
and -fsanitize=undefined on the host compilation only) and runs the host-side
ABI tests against it in a child process, with the clang ASan runtime preloaded
and every sanitizer report fatal.  No GPU is needed: the tests exercise the
argument validation, status codes and exports, which run before any launch.
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_abi_under_asan_and_ubsan():
    sys.path.insert(0, ROOT)
    from route_kv_memory_amd.build import build, sanitizer_runtime

    lib = build(verbose=False, sanitize=True)
    res = subprocess.run(["nm", "-D", lib], capture_output=True, text=True)
    assert "__asan_report" in res.stdout and "__ubsan_handle" in res.stdout, \
        "the library is not instrumented"
    env = dict(os.environ, MKA_LIB=lib, LD_PRELOAD=sanitizer_runtime(),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    cmd = [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
           os.path.join(ROOT, "tests", "test_abi_host.py"),
           os.path.join(ROOT, "tests", "test_layer_host.py")]
    run = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (run.stdout + run.stderr)[-3000:]
    assert run.returncode == 0, f"sanitized host tests failed:\n{tail}"
    assert "ERROR: AddressSanitizer" not in tail and "runtime error:" not in tail, tail
    print(tail.strip().splitlines()[-1])
