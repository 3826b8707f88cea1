"""Host-only check of the C ABI's argument validation under AddressSanitizer
and UndefinedBehaviorSanitizer (no GPU): every library source is compiled with
the sanitizers on its host half only (the device half is compiled as usual and
never runs), linked with tests/host/abi_validation_test.cpp, and run where no
GPU is visible.  The driver calls every entry point with arguments that must
be rejected on the host, sweeps natsl_workspace_size over extreme shapes (an
overflow in the size arithmetic is undefined behaviour and stops the run), and
reads the thread-local error text from eight threads at once."""
import concurrent.futures as cf
import os
import shutil
import subprocess

import pytest

from linear_attention_natsl_amd import build as B

ROOT = os.path.abspath(os.path.join(os.path.dirname(__file__), ".."))
DRIVER = os.path.join(ROOT, "tests", "host", "abi_validation_test.cpp")
CLANG = "/opt/rocm/llvm/bin/clang++"
SAN = "address,undefined"

pytestmark = pytest.mark.skipif(
    __import__("torch").cuda.is_available(), reason="runs the host validation paths where no GPU is visible")


def test_abi_validation_under_asan_ubsan(tmp_path):
    try:
        hipcc = B.hipcc()
    except RuntimeError as e:
        pytest.skip(str(e))
    if not os.path.exists(CLANG):
        pytest.skip("ROCm clang++ not found")
    flags = [f for f in B.FLAGS if f != "-O3"] + ["-O1", "-Xarch_host", f"-fsanitize={SAN}",
                                                  "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-g"]

    def compile_one(src):
        obj = str(tmp_path / (src + ".o"))
        cmd = [hipcc, *flags, *B.FILE_FLAGS.get(src, []), "-c", os.path.join(B.CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, B.SOURCES))
    drv = str(tmp_path / "driver.o")
    r = subprocess.run([CLANG, "-std=c++17", "-O1", "-g", f"-fsanitize={SAN}", "-fno-sanitize-recover=all",
                        "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-c", DRIVER, "-o", drv],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    exe = str(tmp_path / "abi_validation")
    r = subprocess.run([CLANG, f"-fsanitize={SAN}", "-pthread", drv, *objs, "-L/opt/rocm/lib", "-lamdhip64",
                        "-Wl,-rpath,/opt/rocm/lib", "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    if r.returncode == 77:
        pytest.skip(r.stdout.strip())
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert " 0 errors" in r.stdout
