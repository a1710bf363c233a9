"""The C ABI's host code under AddressSanitizer (CPU only).

Runs tests/test_abi.py -- every argument check of every entry point, no
kernel launched -- in a child process against libsgmv_asan.so, the library
with its host code built with -fsanitize=address, the sanitizer runtime
preloaded.  A heap or stack overflow, use-after-free or similar in the
host-side validation, planning or launch set-up fails the run.  The pages
report that shape or rank mismatches end in illegal memory accesses
(Punica walkthrough, omica.com.cn/news/959180, section 5.2); the host side
here must reject such calls cleanly instead.
"""
import os
import subprocess
import sys

import pytest

from segmented_gather_gemv_sgmv_amd import build as hip_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def asan_library():
    lib = hip_build.ASAN_LIBRARY
    if not os.path.exists(lib) or os.path.getmtime(lib) < hip_build.sources_mtime():
        hip_build.build_asan()
    return lib


def test_library_is_instrumented(asan_library):
    data = open(asan_library, "rb").read()
    assert b"__asan_report" in data, "libsgmv_asan.so carries no sanitizer checks"


def test_abi_checks_under_address_sanitizer(asan_library):
    env = dict(os.environ)
    env["LD_PRELOAD"] = hip_build.asan_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["SGMV_LIBRARY"] = asan_library
    proc = subprocess.run(
        [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q",
         "-p", "no:cacheprovider", "-m", "not gpu"],
        cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = proc.stdout + proc.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert proc.returncode == 0, out[-4000:]
    assert " passed" in out
