"""The C-ABI argument validation under AddressSanitizer and UBSan: the
library is rebuilt with both sanitizers on its host code
(`build.py --sanitize`), and the CPU validation tests (tests/test_abi_cpu.py,
which call every entry point with invalid arguments, null pointers,
misaligned pointers and oversized shapes) run against it in a child process
with the sanitizer runtime preloaded.  Any sanitizer report fails the test."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from diffusion_drafted_verification_amd import build as B  # noqa: E402


def test_abi_validation_is_clean_under_asan_and_ubsan():
    if not B.hipcc() or not B.asan_runtime():
        pytest.skip("hipcc or the AddressSanitizer runtime is not available")
    lib = B.build_sanitized(verbose=False)
    env = dict(os.environ, ORTHRUS_LIBRARY=lib, LD_PRELOAD=B.asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:allocator_may_return_null=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py"), "-k", "not one_hip_runtime"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout
