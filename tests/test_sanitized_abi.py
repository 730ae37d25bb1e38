"""The C ABI layer under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

miattn.cpp (argument validation, split choice, size arithmetic, dispatch) is
rebuilt with host-side ASan + UBSan and linked with the ordinary device
objects; the host-side ABI and binding tests then run against that library
in a child process with the sanitizer runtime preloaded. Any invalid memory
access or undefined behaviour in the host code those tests reach aborts the
child, and the test fails.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None
                                and not os.path.exists("/opt/rocm/bin/hipcc"),
                                reason="needs the ROCm toolchain")


@pytest.fixture(scope="module")
def sanitized():
    from exact_io_aware_06_amd import build
    lib = build.build_sanitized(verbose=False)
    return lib, build.asan_runtime()


def test_library_is_instrumented(sanitized):
    lib, _ = sanitized
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report_load" in syms or "__asan_load" in syms
    assert "__ubsan_handle" in syms


def test_abi_tests_pass_under_sanitizers(sanitized):
    lib, rt = sanitized
    env = dict(os.environ, LD_PRELOAD=rt, MIATTN_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    cmd = [sys.executable, "-m", "pytest", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
           "tests/test_abi.py", "tests/test_binding_checks.py", "tests/test_zz_no_alloc.py"]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
