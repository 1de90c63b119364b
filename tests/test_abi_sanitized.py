"""The C ABI's host code (api.cpp) under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

``tests/abi_host_check.cpp`` links api.cpp, unchanged, against stub kernel
launchers and exercises every entry point; this test builds it with g++
``-fsanitize=address,undefined`` (host code only, no device code is
involved) and requires a clean run.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "online_softmax_fa2_amd", "csrc")
ROCM_INCLUDE = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(ROCM_INCLUDE),
                    reason="needs g++ and the ROCm headers")
def test_api_host_code_under_asan_ubsan(tmp_path):
    exe = tmp_path / "abi_host_check"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", CSRC, "-I", ROCM_INCLUDE, os.path.join(CSRC, "api.cpp"),
           os.path.join(ROOT, "tests", "abi_host_check.cpp"), "-o", str(exe), "-pthread"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    env.pop("OSFA_SYNC_CHECK", None)
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "abi host check ok" in run.stdout
    assert "ERROR: AddressSanitizer" not in run.stderr and "runtime error" not in run.stderr, run.stderr
