"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).

abi.cpp (argument validation, workspace carving, launch sequencing) is built
with g++ -fsanitize=address,undefined together with host-only stand-ins of the
kernel launchers (tests/abi_host_stubs.cpp), into a library that needs no
GPU.  A child Python process preloads the sanitizer runtime, points the
binding at that library and runs tests/test_abi_cpu.py (invalid arguments,
zero tokens, symbol exports) and tests/abi_stub_checks.py (valid calls of
every entry point at every workload's size, with the expected launch
sequence).  Any sanitizer report aborts the child and fails the test.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_moe_expert_route_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _asan_runtime():
    gxx = shutil.which("g++")
    if not gxx:
        return None
    out = subprocess.run([gxx, "-print-file-name=libasan.so"], stdout=subprocess.PIPE, text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


@pytest.mark.timeout(600)
def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    asan = _asan_runtime()
    if asan is None or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime_api.h")):
        pytest.skip("g++ with libasan and the HIP headers are needed")
    lib = str(tmp_path / "libmoe_host_sanitized.so")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "abi.cpp"), os.path.join(ROOT, "tests", "abi_host_stubs.cpp"), "-o", lib]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert res.returncode == 0, res.stdout
    runner = ("import sys; sys.path[:0] = [%r, %r]; import sparse_moe_expert_route_amd as m; m.lib_path = %r; "
              "import pytest; sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', '-p', 'no:xdist', %r, %r]))"
              % (ROOT, os.path.join(ROOT, "tests"), lib, os.path.join(ROOT, "tests", "test_abi_cpu.py"),
                 os.path.join(ROOT, "tests", "abi_stub_checks.py")))
    env = dict(os.environ)
    env["LD_PRELOAD"] = asan
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env.pop("PYTEST_XDIST_WORKER", None)
    res = subprocess.run([sys.executable, "-c", runner], cwd=ROOT, env=env, stdout=subprocess.PIPE,
                         stderr=subprocess.STDOUT, text=True, timeout=540)
    tail = "\n".join(res.stdout.splitlines()[-40:])
    assert res.returncode == 0, tail
    assert "passed" in tail and "ERROR: AddressSanitizer" not in res.stdout and "runtime error" not in res.stdout, tail
