"""Host code of the library (block pool, metadata validator, error strings)
built with AddressSanitizer and UndefinedBehaviorSanitizer and driven through
the C ABI by tests/host/pool_sanitize.cpp.  CPU only: g++ builds the host
sources on their own, no device code is involved."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_varlen_reshape_amd", "csrc")
HOST_SOURCES = ["pool.cpp", "validate.cpp", "errors.cpp"]


def test_pool_and_validator_under_asan_and_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ is not installed")
    exe = str(tmp_path / "pool_sanitize")
    flags = ["-std=c++17", "-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all"]
    srcs = [os.path.join(ROOT, "tests", "host", "pool_sanitize.cpp")] + [os.path.join(CSRC, s) for s in HOST_SOURCES]
    b = subprocess.run([gxx, *flags, "-I", os.path.join(ROOT, "include"), "-I", CSRC, *srcs, "-o", exe],
                       capture_output=True, text=True, timeout=600)
    assert b.returncode == 0, b.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "checks passed" in r.stdout
