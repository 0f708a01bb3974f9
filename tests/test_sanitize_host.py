"""The oracle and the host side of the C ABI built with AddressSanitizer and
UndefinedBehaviorSanitizer and run on the CPU (no GPU):

* tests/sanitize/oracle_driver.c calls every oracle entry point on small and
  ragged shapes with exactly sized buffers;
* tests/sanitize/abi_driver.cpp calls every C-ABI entry point with argument
  errors and with valid shapes, against stub launchers
  (tests/sanitize/abi_stubs.cpp), so api.cpp's validation runs alone. Only
  host code is instrumented (each -fsanitize= follows -Xarch_host).

Any sanitizer report fails the run (-fno-sanitize-recover=all)."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
HIPCC = "/opt/rocm/bin/hipcc"


def run(cmd, env=None):
    p = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=300)
    assert p.returncode == 0, f"{' '.join(cmd)}\n{p.stdout}\n{p.stderr}"
    return p.stdout


def test_oracle_under_asan_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_driver")
    run(["gcc", "-std=c11", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-fno-omit-frame-pointer", "-fopenmp", "-ffp-contract=off", os.path.join(SAN, "oracle_driver.c"),
         os.path.join(ROOT, "oracle", "qref.c"), "-o", exe, "-lm"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", OMP_NUM_THREADS="2")
    assert "all calls clean" in run([exe], env)


def test_host_abi_under_asan_ubsan(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "abi_driver")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    run([HIPCC, "--offload-arch=gfx950", "-std=c++17", "-O1", "-g", *san,
         os.path.join(ROOT, "weight_only_quantized_qgemv_amd", "csrc", "api.cpp"),
         os.path.join(SAN, "abi_stubs.cpp"), os.path.join(SAN, "abi_driver.cpp"), "-o", exe])
    # Leak checking is off: the HIP runtime's own start-up allocations would
    # be reported.
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0")
    assert "all calls clean" in run([exe], env)
