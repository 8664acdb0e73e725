"""The C ABI's host code (argument validation in api.cpp) under AddressSanitizer and
UndefinedBehaviorSanitizer: tests/test_abi.py run against a build whose host side is
instrumented, in a child process with the clang ASan runtime preloaded.  No GPU is
needed: every call there is refused on the host before any launch."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_checks_under_host_asan_ubsan():
    from selective_state_space_14_amd import build
    try:
        runtime = build.host_sanitizer_runtime()
    except (RuntimeError, OSError) as e:
        pytest.skip(f"no ASan runtime: {e}")
    lib = build.build_host_sanitized(verbose=False)
    env = dict(os.environ, LD_PRELOAD=runtime, SSD_LIBRARY=lib, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, tail
    assert " passed" in r.stdout, tail
