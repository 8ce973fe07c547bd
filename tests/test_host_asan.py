"""The C ABI layer (csrc/api.cpp with the planning rules of csrc/plan.cpp)
built for the host with AddressSanitizer and UndefinedBehaviorSanitizer
against recording stand-ins of the kernel launchers and of the HIP runtime
(tests/host_asan/): structs of every ABI version read from buffers of exactly
their size, host offset arrays of exactly their length, argument checks that
launch nothing, and the launch sequences the planning rules choose (the
decode gate followed by route_count, routing passes of KV heads, the
entry point that allocates nothing).  CPU only: g++, no GPU, no HIP device
code."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "host_asan")
CSRC = os.path.join(ROOT, "block_sparse_attention_gate_amd", "csrc")


def _rocm_include():
    for cand in ("/opt/rocm/include",):
        if os.path.exists(os.path.join(cand, "hip", "hip_runtime.h")):
            return cand
    return None


def test_abi_layer_under_address_sanitizer(tmp_path):
    gxx = shutil.which("g++")
    inc = _rocm_include()
    if gxx is None or inc is None:
        pytest.skip("needs g++ and the HIP headers")
    exe = str(tmp_path / "host_checks")
    cmd = [gxx, "-std=c++17", "-g", "-O1", "-fsanitize=address,undefined",
           "-fno-omit-frame-pointer", "-fno-sanitize-recover=undefined",
           "-D__HIP_PLATFORM_AMD__", "-I", inc, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "plan.cpp"),
           os.path.join(HERE, "host_stub.cpp"), os.path.join(HERE, "host_checks.cpp"),
           "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    print(run.stdout)
    assert run.returncode == 0 and run.stdout.strip().endswith("passed"), (
        run.stdout[-3000:] + run.stderr[-3000:])
