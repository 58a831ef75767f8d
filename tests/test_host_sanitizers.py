"""The C ABI's host-side validation, workspace carving and launch sequencing (api.cpp) built
with g++ under AddressSanitizer and UndefinedBehaviorSanitizer, with host-only stand-ins for
the kernel launchers (tests/sanitize/stub_launchers.cpp), driven through valid and invalid
arguments (tests/sanitize/drive_abi.cpp). Needs no GPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the ROCm headers")
def test_host_paths_are_clean_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "drive_abi")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           f"-I{ROOT}/include", f"-I{ROOT}/bit_grouped_gemm_amd/csrc",
           f"{ROOT}/bit_grouped_gemm_amd/csrc/api.cpp", f"{ROOT}/tests/sanitize/stub_launchers.cpp",
           f"{ROOT}/tests/sanitize/drive_abi.cpp", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "ok (0 failures)" in r.stdout
