"""Host-side checks of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer, with no device.

api.cpp (validation, workspace plan, launch order, error reporting) is built with g++ against stub launchers and a
stub HIP runtime (tests/host_abi): every launcher records its name and can be made to fail, and so can the runtime
calls the host code makes. tests/host_abi/driver.cpp then checks every validation code of every entry point, the
launch order of each stage, SAGESLA_E_HIP and sagesla_last_hip_error for a failure injected at each launch, the
allocation-free entry point's scratch lookup, and, run with SAGESLA_DEBUG=1, the synchronizing debug mode.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST = os.path.join(ROOT, "tests", "host_abi")
SOURCES = [os.path.join(ROOT, "int8_block_sparse_amd", "csrc", "api.cpp"), os.path.join(HOST, "stubs.cpp"),
           os.path.join(HOST, "driver.cpp")]


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    cxx = shutil.which("g++")
    if not cxx:
        pytest.skip("g++ not found")
    exe = str(tmp_path_factory.mktemp("abi_host") / "abi_host")
    cmd = [cxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-Wall",
           "-Werror", "-I", HOST, "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "int8_block_sparse_amd", "csrc"), *SOURCES, "-o", exe, "-lpthread"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    return exe


def run(exe, debug):
    env = dict(os.environ)
    env.pop("SAGESLA_DEBUG", None)
    if debug:
        env["SAGESLA_DEBUG"] = "1"
    env["ASAN_OPTIONS"] = "abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    return subprocess.run([exe] + (["debug"] if debug else []), capture_output=True, text=True, timeout=300, env=env)


def test_validation_launch_order_and_hip_errors(driver):
    r = run(driver, debug=False)
    assert r.returncode == 0, r.stdout + r.stderr[-4000:]
    assert "host ABI checks passed" in r.stdout and "(default mode)" in r.stdout
    assert "sagesla:" not in r.stderr  # without the debug mode nothing is printed


def test_debug_mode_synchronizes_each_stage(driver):
    r = run(driver, debug=True)
    assert r.returncode == 0, r.stdout + r.stderr[-4000:]
    assert "(debug mode)" in r.stdout
    # each injected fault is named with the launcher of its stage
    for name in ("launch_kmean", "launch_quant", "launch_scores", "launch_topk", "launch_linear", "launch_attn",
                 "launch_backward_sparse", "launch_w8a8_gemm"):
        assert f"sagesla: {name}: injected error" in r.stderr, name
