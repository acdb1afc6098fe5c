"""The library's host-side planning (tile lists, band rasters, XCD segments,
longest-first layouts, the persistent chain's queues and completion counts),
checked on the CPU by host_plan/plan_check.cpp: muon_api.cpp compiled for the
host with the HIP runtime replaced by host-memory stubs and the kernel
launchers replaced by checkers that walk the device lists as the kernels do.
Built with address and undefined-behaviour sanitizers."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
HIP_INC = "/opt/rocm/include"


@pytest.fixture(scope="module")
def plan_check(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists(os.path.join(HIP_INC, "hip", "hip_runtime.h")):
        pytest.skip("needs g++ and the HIP headers")
    exe = tmp_path_factory.mktemp("plan") / "plan_check"
    cmd = [gxx, "-std=c++17", "-O1", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I", HIP_INC,
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "muon_newton_schulz_02_amd", "csrc"),
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-o", str(exe), os.path.join(HERE, "host_plan", "plan_check.cpp")]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    return exe


def test_tile_walks_and_chain_queues(plan_check):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0")
    r = subprocess.run([str(plan_check)], capture_output=True, text=True, timeout=600, env=env)
    out = r.stdout
    assert r.returncode == 0 and "PLAN-CHECK OK" in out and "FAIL" not in out, out[-6000:] + r.stderr[-3000:]
    # the d24 stack: 144 matrices, 6 x 6 tile rows and columns (square) or
    # 6 x 24 (rectangular): 21 triangle tiles each for GRAM and POLY
    d24 = out.split("CASE grids d24 stack")[1].split("CASE")[0]
    assert d24.count(" 3024 tiles") == 2 and " 10368 tiles" in d24
    assert out.count("CASE ") == 15
    assert "out of memory with the hook, launched without it" in out
    # the allocation-free entry point: buffers and tables inside its scratch
    # block, and a stack too large for it refused before any launch
    assert out.count("CASE no-allocation") == 3
    big_na = out.split("CASE no-allocation one d24 layer (too large)")[1].split("CASE")[0]
    assert "status 2" in big_na and "fixed" in big_na
    # formats: one 256 x 256 binary32 matrix on 64 x 64 tiles (4 x 4: 10
    # triangle tiles, 16 product tiles); the larger binary32 stack on 128 x 128
    one = out.split("CASE grids single 256 x 256")[1].split("CASE")[0]
    assert "phase 0 prec 4: 10 tiles" in one and "phase 2 prec 4: 16 tiles" in one
    big = out.split("CASE grids binary32 stack on 128 x 128 tiles")[1].split("CASE")[0]
    assert "phase 0 prec 2:" in big and "prec 4" not in big
    # split-bf16: eight 2048^2 matrices fill the GPU with 256 x 256 tiles (8 x 9 / 2
    # = 36 triangle tiles each; format 1), the two small ones of the ragged
    # case run on 128 x 128 tiles (format 5)
    x3 = out.split("CASE grids split-bf16 stack on 256 x 256 tiles")[1].split("CASE")[0]
    assert "phase 0 prec 1: 288 tiles" in x3 and "prec 5" not in x3
    ragged = out.split("CASE grids ragged, mixed formats")[1].split("CASE")[0]
    assert "prec 5" in ragged and "prec 1:" not in ragged
    assert out.count("  chain prec ") == 5
