"""Host builds with AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The fp64 oracle (oracle/oracle.c) linked into tests/sanitize/oracle_driver.c,
  which runs every oracle routine on small seeded inputs.
* The C ABI's argument checks (api.cpp), with the kernel launchers and the HIP
  runtime queries replaced by host stubs (tests/sanitize/abi_stubs.cpp), driven
  through every entry point by tests/sanitize/abi_driver.cpp.

Any out-of-bounds access, leak, integer overflow, invalid enum load or
misaligned access aborts the run with a sanitizer report.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
FLAGS = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-fno-omit-frame-pointer"]


def _run(exe):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_asan")
    subprocess.run(["gcc", "-std=gnu11", *FLAGS, "-fopenmp", "-Wall", "-Wextra",
                    os.path.join(SAN, "oracle_driver.c"), os.path.join(ROOT, "oracle", "oracle.c"),
                    "-lm", "-o", exe], check=True, timeout=120)
    assert "oracle driver ok" in _run(exe)


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="g++ or the HIP headers not available")
def test_c_abi_checks_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "abi_asan")
    subprocess.run(["g++", "-std=c++17", *FLAGS, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    "-Wall", os.path.join(SAN, "abi_driver.cpp"), os.path.join(SAN, "abi_stubs.cpp"),
                    os.path.join(ROOT, "affine_quantized_gemv_qgemv_amd", "csrc", "api.cpp"),
                    "-o", exe], check=True, timeout=180)
    assert "abi driver ok" in _run(exe)
