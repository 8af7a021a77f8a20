"""The C ABI's host code under the address and undefined-behaviour sanitizers (CPU only).

llp_api.cpp (request validation, workspace layout, launch sequences) is built with the host
compiler and -fsanitize=address,undefined against tests/sanitize/hip_stub.cpp, a stand-in HIP
runtime whose launchers touch the first and last element of every array each kernel would
address, and driven by tests/sanitize/abi_cases.cpp: malformed requests must be refused with the
documented status; well-formed ones for every entry point must address only the exactly sized
buffers they were given. A sanitizer report or a wrong status fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = [os.path.join(ROOT, "lm_head_linear_logp_amd", "csrc", "llp_api.cpp"),
       os.path.join(ROOT, "tests", "sanitize", "hip_stub.cpp"),
       os.path.join(ROOT, "tests", "sanitize", "abi_cases.cpp")]
HIP_INCLUDE = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(HIP_INCLUDE),
                    reason="needs g++ and the HIP headers")
def test_host_code_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "abi_cases")
    cmd = ["g++", "-std=c++17", "-g", "-O1", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", f"-I{ROOT}/include",
           f"-I{ROOT}/lm_head_linear_logp_amd/csrc", f"-I{HIP_INCLUDE}", *SRC, "-o", exe]
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert b.returncode == 0, b.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-6000:]
    assert "Sanitizer" not in out and "runtime error" not in out, out[-6000:]
    assert " 0 failed" in out, out[-2000:]
