"""The decode plan's invariants, checked on the host (no GPU): tests/plan_check.cpp
is compiled with g++ against the planner's own header and sweeps shapes,
lengths up to the length cap, windows and partition sizes (grid splits hold
at most 64 pages per wave, balanced ranges at most 64 * W pages, no item
meets more ranges than it has partial slots, the workspace's counter region
sits at offset 0 and does not move with the shape)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_plan_invariants(tmp_path):
    exe = tmp_path / "plan_check"
    src = os.path.join(ROOT, "tests", "plan_check.cpp")
    subprocess.run(["g++", "-O2", "-std=c++17", "-Wall", "-Werror", src, "-o", str(exe)],
                   check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok ")
