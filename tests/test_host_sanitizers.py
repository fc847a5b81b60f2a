"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

* The oracle (oracle/kdn_oracle.c) is built with -fsanitize=address,undefined
  and the oracle pin tests are run against that build in a child process, so
  an out-of-bounds access or undefined behaviour anywhere in the oracle fails
  them.  The AddressSanitizer runtime has to be loaded before the
  interpreter, so the child gets it through LD_PRELOAD; the test is skipped
  where LD_PRELOAD is already set by the environment (nothing of it is
  replaced).
* The C ABI's host side (kdn_api.cpp: validation, workspace layout, the order
  and arguments of the launches) is built with a host compiler alone, linked
  with tests/abi_host_driver.cpp, whose stubs stand in for the kernel
  launchers and check every workspace buffer they are handed, and run under
  the same sanitizers.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]


def _runtime(name: str) -> str | None:
    out = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                         text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


@pytest.fixture(scope="module")
def tmp(tmp_path_factory):
    return tmp_path_factory.mktemp("sanitizers")


def test_oracle_pins_pass_under_address_and_undefined_behaviour_sanitizers(tmp):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    if os.environ.get("LD_PRELOAD"):
        pytest.skip("LD_PRELOAD is already set by the environment")
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("no AddressSanitizer runtime")
    lib = str(tmp / "_kdn_oracle_asan.so")
    subprocess.check_call(["gcc", "-std=c99", "-fPIC", "-shared", "-pthread", *SAN,
                           os.path.join(ROOT, "oracle", "kdn_oracle.c"), "-o", lib])
    env = dict(os.environ, KDN_ORACLE_LIB=lib, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    pins = ["tests/test_oracle_pins.py", "tests/test_oracle_grad_pins.py",
            "tests/test_oracle_dense_pins.py", "tests/test_oracle_golden.py",
            "tests/test_oracle_layer_pins.py"]
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu",
                          "-p", "no:cacheprovider", *pins], cwd=ROOT, env=env,
                         capture_output=True, text=True, timeout=900)
    out = res.stdout + res.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    assert " passed" in res.stdout


def test_c_abi_host_side_under_address_and_undefined_behaviour_sanitizers(tmp):
    if shutil.which("g++") is None:
        pytest.skip("g++ not found")
    if not os.path.exists("/opt/rocm/include/hip/hip_runtime_api.h"):
        pytest.skip("HIP headers not found")
    exe = str(tmp / "abi_host_driver")
    subprocess.check_call(
        ["g++", "-std=c++17", "-Wall", "-Wno-attributes", "-Wno-unused-function",
         "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
         "-I", os.path.join(ROOT, "kalman_filter_memory_amd", "csrc"), *SAN,
         os.path.join(ROOT, "kalman_filter_memory_amd", "csrc", "kdn_api.cpp"),
         os.path.join(ROOT, "tests", "abi_host_driver.cpp"), "-o", exe],
        stderr=subprocess.DEVNULL)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([exe], env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "0 failures" in res.stdout
