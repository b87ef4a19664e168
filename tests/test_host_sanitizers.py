"""The library's host code (ra_api.cpp: validation, workspace layouts,
launch sequences, the graph build, the layer budgets) built with g++ under
AddressSanitizer and UndefinedBehaviorSanitizer, with the kernel launchers
and the HIP runtime calls stubbed, and run on the CPU
(tests/native/host_checks.cpp says what it checks)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "host_checks")


def test_host_code_under_asan_and_ubsan():
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ is not installed")
    os.makedirs(os.path.dirname(OUT), exist_ok=True)
    flags = ["-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
             "-D__align__(n)=__attribute__((aligned(n)))",
             "-DHIP_SYMBOL(x)=((const void*)&(x))",
             "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
             "-I" + os.path.join(ROOT, "top_sparse_attention_gqa_amd", "csrc")]
    srcs = [os.path.join(ROOT, "top_sparse_attention_gqa_amd", "csrc", "ra_api.cpp"),
            os.path.join(ROOT, "tests", "native", "host_checks.cpp")]
    r = subprocess.run([gxx, *flags, *srcs, "-o", OUT], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([OUT], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "host checks ok" in r.stdout
