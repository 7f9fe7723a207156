"""The C ABI's host code (api.cpp and the dispatch helpers) built with the address and
undefined-behaviour sanitizers and driven by tests/abi_host/check_abi.cpp against
stand-in launchers: rejected calls request no launch, accepted calls request the
expected launches, and a launch the runtime rejects comes back as NVFP4_EHIP (also
after an earlier kernel of the same call was enqueued).  Host only: g++ builds it,
no device code is involved."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "nvfp4_w4a4_block_act_amd", "csrc")
HOST = os.path.join(ROOT, "tests", "abi_host")
ROCM_INCLUDE = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "include")


def test_c_abi_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir(ROCM_INCLUDE):
        pytest.skip("g++ or the HIP runtime headers are not available")
    exe = str(tmp_path / "check_abi")
    sources = [os.path.join(HOST, "check_abi.cpp"), os.path.join(HOST, "stub_launchers.cpp"),
               os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "dispatch.cpp")]
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-Wall", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-static-libasan",
           "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INCLUDE, *sources, "-o", exe]
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert b.returncode == 0, b.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0, (r.stdout[-4000:], r.stderr[-4000:])
    assert r.stdout.strip().splitlines()[-1].startswith("ok "), r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]


def test_launch_rules_host(tmp_path):
    """The launch rules of launch.hpp (wave count of the weight-streaming kernels,
    one-launch row bounds and tiles per wave, MFMA tiling choice): documented
    values, and a kernel instance for every (M, K) the one-launch layer accepts
    over a sweep of K and N (tests/abi_host/check_policy.cpp)."""
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir(ROCM_INCLUDE):
        pytest.skip("g++ or the HIP runtime headers are not available")
    exe = str(tmp_path / "check_policy")
    cmd = [gxx, "-std=c++17", "-O1", "-Wall", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
           "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INCLUDE, os.path.join(HOST, "check_policy.cpp"), "-o", exe]
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert b.returncode == 0, b.stderr[-4000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout[-4000:]
    assert r.stdout.strip().splitlines()[-1].startswith("ok "), r.stdout
