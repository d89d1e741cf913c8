"""The inbox guard's bookkeeping on the CPU (no GPU).

tests/guard_units_check.cpp compiles the kernels' and the host library's own
header (shard_decomposed_gemm_amd/csrc/guard_units.h) with g++ and checks that
the totals the host keeps for a producer's wait equal what the consumers'
units count into each counter, for every launch size up to 4096 units and a
few large ones, and over 500 launches that take the 32-bit counters across
their wrap. A planted mistake in the totals must fail it.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "guard_units_check.cpp")
INC = os.path.join(ROOT, "shard_decomposed_gemm_amd", "csrc")


def _build(tmp_path, plant=0):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path / f"guc{plant}")
    subprocess.run([gxx, "-O2", "-std=c++17", "-Wall", f"-DPLANT={plant}", "-I", INC, SRC, "-o", exe], check=True)
    return exe


def test_guard_totals_match_the_counts(tmp_path):
    r = subprocess.run([_build(tmp_path)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok:"), r.stdout


def test_planted_mistake_in_the_totals_is_caught(tmp_path):
    r = subprocess.run([_build(tmp_path, 1)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 1 and r.stdout.startswith("FAIL:"), r.stdout
