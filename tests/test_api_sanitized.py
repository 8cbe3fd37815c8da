"""The C ABI's host-side argument checks (csrc/api.cpp) built with g++ under
AddressSanitizer and UndefinedBehaviorSanitizer, against stub launchers: every entry point
returns its documented status for invalid arguments without enqueuing anything, and hands
valid arguments to its launcher (no GPU needed)."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
DRIVER = os.path.join(HERE, "native", "api_checks.cpp")
API = os.path.join(ROOT, "fp4_w8a8_quantized_amd", "csrc", "api.cpp")


def test_api_checks_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("g++ or the ROCm headers not available")
    out = str(tmp_path / "api_checks")
    flags = ["-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
             "-I" + os.path.join(ROOT, "include")]
    subprocess.run([gxx, *flags, DRIVER, API, "-o", out], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([out], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failures" in r.stdout, r.stdout
