"""The GEMM launch planner's host logic, without a GPU: tests/c/plan_check.hip compiles
gemm_plan.hip for the host with stub launchers and checks the 256-row / 192-row cut (every column
strip's rows covered exactly once, each launch within its rounds, no cut for whole or short last
rounds, the planned cut of the 4096 x 3584 SiLU·up launch), the four-wave kernel's tile map (a
bijection for every group height), the L2 fetch count that picks the group heights (the
figures the FETCH_SIZE counters confirmed on the device), and which kernel the 70B TP=8 prefill
GEMMs run on (the 16 x 16 x 32 kernel, for [k][n] and [n][k] weights)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC") or ("/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else shutil.which("hipcc"))


@pytest.mark.skipif(HIPCC is None, reason="needs hipcc")
def test_launch_planner_host_logic(tmp_path):
    exe = tmp_path / "plan_check"
    cmd = [HIPCC, "-std=c++20", "-O1", "-I", os.path.join(ROOT, "tensor_transformer_linear_amd", "csrc"),
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c", "plan_check.hip"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "ALL OK" in out.stdout
