"""The library's host layer (argument validation, launch planning, error
propagation; abi.cpp and plan.cpp) built for the CPU with AddressSanitizer and
UndefinedBehaviorSanitizer against a stand-in device side
(tests/host_abi/stub_device.cpp), then run: launch failures reach the caller
as MOE_ERR_HIP, errors the caller left pending are not reported as the call's
own, validation failures launch nothing, error details are per thread."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "quantized_moe_expert_top_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "host_abi")


def test_host_layer_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no g++")
    exe = str(tmp_path / "host_abi_test")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
           "-fno-sanitize-recover=all", "-Wall", "-Wextra", "-Wno-unused-parameter", "-Werror",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", HERE,
           os.path.join(CSRC, "abi.cpp"), os.path.join(CSRC, "plan.cpp"),
           os.path.join(HERE, "stub_device.cpp"), os.path.join(HERE, "host_abi_test.cpp"), "-o", exe, "-pthread"]
    subprocess.run(cmd, check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "host layer checks passed" in r.stdout
