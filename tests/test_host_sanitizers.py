"""The C-ABI host layer (validation, planner, launch arguments) built with g++
under AddressSanitizer and UndefinedBehaviorSanitizer against host-only stubs
of the HIP runtime and the kernel launchers, and exercised by a C++ driver.
No GPU is touched: the stubs record the launches the calls would make."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "host_abi")
CSRC = os.path.join(ROOT, "decode_attention_paged_06_amd", "csrc")
ROCM_INCLUDE = "/opt/rocm/include"


def test_host_layer_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir(ROCM_INCLUDE):
        pytest.skip("needs g++ and the ROCm headers")
    exe = str(tmp_path / "host_abi")
    cmd = [gxx, "-std=c++17", "-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM_INCLUDE}",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", f"-I{HERE}",
           os.path.join(CSRC, "host", "api.cpp"), os.path.join(HERE, "hip_stubs.cpp"),
           os.path.join(HERE, "driver.cpp"), "-o", exe, "-lpthread"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([exe], capture_output=True, text=True, env=env)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "all checks passed" in res.stdout
