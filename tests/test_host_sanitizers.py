"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

tests/host_abi_driver.cpp replaces the kernel launchers and the few HIP runtime calls of the C-ABI
file with counting stubs and drives every entry point through its argument-error cases (status
returned, nothing launched) and through valid calls with fake device pointers (the whole host
path: checks, shape planning, workspace carving, the launch sequence).  It is built with g++ and
the host sanitizers only; no device code is involved."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "spec_verify_cad_amd", "csrc")
ROCM_INC = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(ROCM_INC), reason="needs g++ and the HIP headers")
def test_c_abi_host_code_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "abi_sanitized")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", f"-I{ROOT}/include", f"-I{CSRC}", f"-I{ROCM_INC}",
           os.path.join(CSRC, "cad_api.cpp"), os.path.join(ROOT, "tests", "host_abi_driver.cpp"), "-o", exe]
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert b.returncode == 0, b.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0 and "all cases passed" in r.stdout, (r.stdout[-4000:], r.stderr[-4000:])
