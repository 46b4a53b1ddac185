"""The host planner built with AddressSanitizer and UndefinedBehaviorSanitizer
(g++, host code only) and run over random groups: every table the kernels
read stays inside the bounds they rely on (tests/host/plan_invariants.cpp
lists the checks).  CPU only; no device call is made."""

from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "muon_newton_schulz_step_amd", "csrc")
ROCM_INCLUDE = "/opt/rocm/include"


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir(ROCM_INCLUDE):
        pytest.skip("g++ or the ROCm headers are not available")
    out = tmp_path_factory.mktemp("planner_asan")
    exe = str(out / "plan_invariants")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-I", ROCM_INCLUDE, os.path.join(CSRC, "plan.cpp"), os.path.join(ROOT, "tests", "host", "plan_invariants.cpp"),
           "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_planner_invariants_under_sanitizers(checker, seed):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1", UBSAN_OPTIONS="halt_on_error=1")
    r = subprocess.run([checker, str(seed), "150"], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "plan invariants ok" in r.stdout
    # the random groups include large-tile blocks under the persistent schedule
    queued = int(r.stdout.split("plans, ")[1].split()[0])
    assert queued > 0, r.stdout
