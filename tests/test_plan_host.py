"""Host-side arithmetic of the planner, compiled with g++ (no GPU): the
multiply-shift division by launch constants and the tile order built on it
(every tile id maps to one in-range tile, exactly once, in the documented
order), the two-level batch split, the LDS row pads (every kernel's
fragment reads and staging writes free of bank conflicts under gfx950's
lane groups), and the fused attention kernel's key-block layout (each
fragment read finds what the staging wrote, the kernel's base-plus-constant
addressing matches the layout, and every access is conflict-free)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "strided_fp32_gemm_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_planner_host_arithmetic(tmp_path):
    exe = tmp_path / "plan_check"
    subprocess.run(["g++", "-O2", "-std=c++17", "-Wall", "-I", CSRC,
                    os.path.join(HERE, "plan_check.cpp"), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr
