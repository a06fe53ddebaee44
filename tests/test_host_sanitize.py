"""The C ABI's validation paths under AddressSanitizer and
UndefinedBehaviorSanitizer, on the host: fa_api.cpp and fa_host.cpp built
with g++ (no device code), the launchers and HIP runtime calls replaced by
host stand-ins (tests/host_sanitize/stubs.cpp) that check what a kernel
would receive, driven by boundary values of every argument and a seeded
random mix of them (tests/host_sanitize/driver.cpp).  Any sanitizer report
aborts the run."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "io_aware_transformer_amd", "csrc")
ROCM_INC = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(ROCM_INC), reason="needs g++ and HIP headers")
def test_abi_validation_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "fa_host_sanitize")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INC, "-I", os.path.join(ROOT, "include"),
           "-I", CSRC, os.path.join(CSRC, "fa_api.cpp"), os.path.join(CSRC, "fa_host.cpp"),
           os.path.join(HERE, "host_sanitize", "stubs.cpp"), os.path.join(HERE, "host_sanitize", "driver.cpp"),
           "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe, "1000000"], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "0 failures" in run.stdout
