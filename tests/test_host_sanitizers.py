"""The host logic's CPU tests, rerun against an AddressSanitizer + UBSan
build of the same sources (ring.cpp, plan.cpp and the recording launcher),
in a child process that preloads the ASan runtime.  Any out-of-bounds access,
use after free or undefined behaviour in the host code fails the run."""
import os
import subprocess
import sys

import pytest

from chunked_attention_amd import build as kbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_logic_under_asan_and_ubsan():
    kbuild.build_host(sanitize=True)
    rt = kbuild.asan_runtime()
    if not os.path.exists(rt):
        pytest.skip(f"no ASan runtime at {rt}")
    env = dict(os.environ)
    env["LD_PRELOAD"] = rt
    env["KVC_HOST_SANITIZE"] = "1"
    # the interpreter itself is not instrumented: its allocations at exit are
    # not leaks of the code under test
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_host_ring.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
