"""The C-ABI host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): builds the host-instrumented library (device code as usual) and
runs the ABI tests against it in a child process that preloads clang's
sanitizer runtime, halting on the first report."""
import os
import shutil
import subprocess
import sys

import pytest

from block_sparse_attention_scores_amd import build as BUILD

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def sanitized():
    try:
        BUILD.hipcc()
        runtime = BUILD.sanitizer_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    return BUILD.build_sanitized(verbose=False), runtime


def test_library_is_instrumented(sanitized):
    lib, _ = sanitized
    nm = shutil.which("nm")
    if not nm:
        pytest.skip("nm not found")
    syms = subprocess.run([nm, "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms


def test_abi_tests_pass_under_sanitizers(sanitized):
    lib, runtime = sanitized
    env = dict(os.environ, LD_PRELOAD=runtime, SA_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out
    assert " passed" in out
