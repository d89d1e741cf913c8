"""The MFMA consumer's integer schedule on the CPU (no GPU).

tests/mfma_sched_check.cpp compiles the kernel's own schedule header
(shard_decomposed_gemm_amd/csrc/mfma_sched.h) with g++ and replays every
workgroup's compute walk and direct-load cursor over hundreds of shapes, grid
sizes, flag tilings and split / whole-tile / arrival modes, checking that each
k-step of each output tile is computed once and loaded from the right shard
buffer and B rows, that every lane's 16-byte load is in bounds, and that no
flag tile is read before its gate. Two planted mistakes must be caught.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "mfma_sched_check.cpp")
INC = os.path.join(ROOT, "shard_decomposed_gemm_amd", "csrc")


def _build(tmp_path, plant=0):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path / f"msc{plant}")
    subprocess.run([gxx, "-O2", "-std=c++17", "-Wall", f"-DPLANT={plant}", "-I", INC, SRC, "-o", exe], check=True)
    return exe


def test_schedule_covers_every_step_once_in_bounds_and_gated(tmp_path):
    exe = _build(tmp_path)
    r = subprocess.run([exe, "400"], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok: 400 shapes"), r.stdout


@pytest.mark.parametrize("plant,what", [(1, "before its gate"), (2, "load ")])
def test_planted_schedule_mistakes_are_caught(tmp_path, plant, what):
    exe = _build(tmp_path, plant)
    r = subprocess.run([exe, "40"], capture_output=True, text=True, timeout=600)
    assert r.returncode == 1, r.stdout
    assert "FAIL" in r.stdout and what in r.stdout, r.stdout
