"""Host-only concurrency test of the helper-context pool behind natsl_forward
(no GPU): tests/host/helper_pool_test.cpp built with g++ under
ThreadSanitizer, then under AddressSanitizer + UBSan, and run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.abspath(os.path.join(os.path.dirname(__file__), ".."))
SRC = os.path.join(ROOT, "tests", "host", "helper_pool_test.cpp")


@pytest.mark.parametrize("san", ["thread", "address,undefined"])
def test_helper_pool_concurrent_leases(tmp_path, san):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = tmp_path / "pool_test"
    r = subprocess.run([gxx, "-std=c++17", "-O1", "-g", "-pthread", f"-fsanitize={san}", "-fno-sanitize-recover=all",
                        SRC, "-o", str(exe)], capture_output=True, text=True)
    if r.returncode != 0 and "sanitizer" in r.stderr.lower() and "not" in r.stderr.lower():
        pytest.skip(f"{san} sanitizer unavailable: {r.stderr[-300:]}")
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1", ASAN_OPTIONS="detect_leaks=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 errors" in r.stdout
