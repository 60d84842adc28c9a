"""The C ABI's host code (argument validation, top-k chunking, attention
key-range splits and workspace sizing in csa_abi.cpp) built with g++ under
AddressSanitizer and UndefinedBehaviorSanitizer, with host-only stand-ins
for the kernel launchers (tests/c_abi/launch_stubs.cpp), and driven over
thousands of random shapes by tests/c_abi/validate_host.cpp.  CPU only: no
device memory is touched."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = "/opt/rocm"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(os.path.join(ROCM, "include", "hip")),
                    reason="needs g++ and the ROCm headers")
def test_host_abi_under_asan_and_ubsan():
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "validate_host")
        cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
               "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", f"-I{ROOT}/include",
               f"-I{ROOT}/sparse_compressed_attention_amd/csrc", f"-I{ROOT}/tests/c_abi",
               f"{ROOT}/sparse_compressed_attention_amd/csrc/csa_abi.cpp", f"{ROOT}/tests/c_abi/launch_stubs.cpp",
               f"{ROOT}/tests/c_abi/validate_host.cpp", f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib",
               "-o", exe]
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stdout + res.stderr
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1", UBSAN_OPTIONS="halt_on_error=1")
        res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
        out = res.stdout + res.stderr
        assert res.returncode == 0, out
        assert "runtime error" not in out and "AddressSanitizer" not in out, out
        assert "0 failures" in res.stdout
