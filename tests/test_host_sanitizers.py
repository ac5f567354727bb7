"""The host side of the C ABI (argument validation, workspace layout, launch
sequence) built with g++ under AddressSanitizer and UndefinedBehaviorSanitizer
and run with recording stubs in place of the kernel launchers (CPU only)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(os.path.join(ROCM, "include", "hip")),
                    reason="needs g++ and the HIP headers")
def test_host_validator_under_sanitizers(tmp_path):
    exe = str(tmp_path / "host_validator")
    cmd = ["g++", "-std=c++17", "-w", "-g", "-O1", "-D__HIP_PLATFORM_AMD__",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "moe_speculative_decoding_router_amd", "csrc"),
           "-I", os.path.join(ROOT, "tests", "host"),
           os.path.join(ROOT, "moe_speculative_decoding_router_amd", "csrc", "moe_verify.cpp"),
           os.path.join(ROOT, "tests", "host", "stub_launch.cpp"),
           os.path.join(ROOT, "tests", "host", "validate_main.cpp"),
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "all checks passed" in r.stdout
