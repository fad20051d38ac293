"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The HIP library's host code (problem resolution, argument and workspace
checks, chain tables, launch set-up) and the C oracle are rebuilt with both
sanitizers (device code is not instrumented), and the CPU tests that exercise
them -- the boundary's validation, the exported symbols and the oracle's pins
-- run again in a child process with clang's ASan runtime preloaded.  Any
out-of-bounds access, use after free or undefined behaviour (signed overflow,
bad shifts, misaligned loads) aborts the child and fails this test.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


@pytest.mark.skipif(_asan_runtime() is None, reason="clang's ASan runtime is not installed")
def test_host_code_and_oracle_under_asan_ubsan(tmp_path):
    sys.path.insert(0, ROOT)
    from chunked_gated_delta_gdn_amd import _build
    import oracle.build as obuild
    out = os.path.join(ROOT, "_build", "sanitize")
    lib = _build.build_sanitized(out)
    olib = obuild.build_sanitized(os.path.join(out, "liboracle_sanitized.so"))
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": _asan_runtime(),
        "GDN_LIBRARY": lib,
        "GDN_ORACLE_LIBRARY": olib,
        # Python and torch are not instrumented: leaks are theirs, and their
        # allocations stay out of the checks
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    tests = ["tests/test_host_validation.py", "tests/test_abi.py", "tests/test_oracle_pins.py"]
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
                        *tests], cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout, tail
