"""The C-ABI layer (abi.cpp) built for the host with g++ under
AddressSanitizer and UndefinedBehaviorSanitizer, with stand-in launchers that
enqueue nothing and instead check every launch the layer builds: each
workspace operand of every kernel (Newton-Schulz GEMM stages, pack, momentum
partials) must lie inside the caller's workspace over its whole extent.  The
driver runs every entry point through valid and invalid arguments, including
the benchmark workloads' shapes (fake device addresses, never dereferenced)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "matrix_aware_optimizer_step_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "host_abi")


def test_abi_layer_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("needs g++ and the ROCm headers")
    exe = tmp_path / "abi_sanitized"
    cmd = [gxx, "-std=c++17", "-g", "-O1", "-Wall", "-Werror", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I", CSRC, "-I", os.path.join(ROOT, "include"), os.path.join(CSRC, "abi.cpp"),
           os.path.join(HERE, "stub_launchers.cpp"), os.path.join(HERE, "driver.cpp"), "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120, env=env)
    assert out.returncode == 0, out.stderr[-4000:]
    assert out.stdout.startswith("ok: ")
