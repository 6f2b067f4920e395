"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/abi_host_check.cpp links api.cpp with replacements for the kernel
launchers and the two device queries it makes, so the argument checks, the
split plan and the marshalling of launch arguments run without a GPU, each
would-be launch recorded. The driver checks that refused calls launch
nothing, that accepted calls launch once with the planned split count and the
caller's workspace, the plan's invariants over a grid of shapes including the
extremes of every int argument, and that no size computation overflows
(signed overflow traps under UBSan; unsigned sizes are compared with 128-bit
arithmetic).
"""

import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang++"


@pytest.mark.skipif(not os.path.exists(CLANG), reason="ROCm clang++ not found")
def test_abi_host_code_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_host_check")
    cmd = [CLANG, "-std=c++17", "-g", "-O1", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "local_linear_attention_amd", "csrc"),
           os.path.join(ROOT, "local_linear_attention_amd", "csrc", "api.cpp"),
           os.path.join(ROOT, "tests", "abi_host_check.cpp"), "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="exitcode=3:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0, (run.stdout[-4000:] + run.stderr[-4000:])
    assert run.stdout.strip().endswith("ok (0 failures)")
