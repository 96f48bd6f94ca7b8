"""The C-ABI validation tests (tests/test_abi.py) run once more against a
build whose host code carries AddressSanitizer and UndefinedBehaviorSanitizer
(long_context_sparse_csa2_amd/build_asan.py), in a child python with the
ASan runtime preloaded: every argument check, error string and workspace
computation runs without a memory or undefined-behaviour error.  CPU only
(the validation returns before any HIP call)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_validation_under_sanitizers(tmp_path):
    from long_context_sparse_csa2_amd import build_asan
    try:
        lib = build_asan.build(str(tmp_path))
        rt = build_asan.runtime()
    except RuntimeError as e:                 # no hipcc / runtime in this image
        pytest.skip(str(e))
    env = dict(os.environ, CSA2_LIB=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in out
