"""The library's host code (argument checks, split plans, workspace layouts)
built with g++ under AddressSanitizer and UndefinedBehaviorSanitizer and run
against every entry point (tests/sanitize/host_abi_sanitize.cpp).  The kernel
launchers are host stubs that touch every workspace and output byte the
kernels would, so a layout or planning mistake is a heap overflow or a failed
check.  No GPU and no HIP compiler are involved."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "decode_attention_lrkv_amd", "csrc")


def test_host_code_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    if not shutil.which("g++") or not os.path.exists("/opt/rocm/include/hip/hip_runtime.h"):
        pytest.skip("needs g++ and the HIP headers")
    exe = str(tmp_path / "host_abi_sanitize")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           os.path.join(CSRC, "lrkv_host.cpp"), os.path.join(ROOT, "tests", "sanitize", "host_abi_sanitize.cpp"),
           "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-6000:]
    assert "host ABI checks passed" in r.stdout
