"""Writes the stored expected values under tests/golden/ from the CPU oracle.

Run from the repository root: ``python tests/golden/make_golden.py``. It calls
only ``oracle`` (and ``synth`` for the seeded inputs); no value comes from the
GPU path.

* ``tiny_w8_m8_k512_n256.txt``: C of the tiny AG+GEMM workload (W = 8,
  M = 8, K = 512, N = 256; "Eliminating Multi-GPU Performance Taxes" analysis
  page, core identity C = sum_s A_s . B[sK/W:(s+1)K/W, :]). Inputs are fp16
  uniform in [-1, 1] from seeds 0xA001 (A) and 0xB001 (B). Every input is a
  multiple of 2^-24 and every running sum of this workload stays below 2^5,
  so the binary64 oracle is exact here and C * 2^48 is an integer: the file
  stores those integers, one output row per line.
* ``fd_w4_h16_d64.txt``: O of the Flash-Decode global reduction (same page,
  Flash Decode global reduction) for W = 4 ranks, H = 16 heads, d = 64, from
  ``synth.fd_partials(0x7A00, 4, 16, 64)``; binary64 values written exactly
  (``float.hex``), one head per line.
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402
from oracle import fd as fdo  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))

TINY = dict(W=8, M=8, K=512, N=256, seed_a=0xA001, seed_b=0xB001)
FD = dict(W=4, H=16, D=64, seed=0x7A00)


def tiny_inputs():
    t = TINY
    a = synth.matrix_f16(t["seed_a"], t["M"], t["K"])
    b = synth.matrix_f16(t["seed_b"], t["K"], t["N"])
    return a, synth.shards(a, t["W"]), b


def fd_inputs():
    return synth.fd_partials(FD["seed"], FD["W"], FD["H"], FD["D"])


def bits_sum(x: np.ndarray) -> int:
    return int(x.astype(np.uint64).sum())


def write_tiny():
    a, sh, b = tiny_inputs()
    c = oracle.sharded_gemm(sh, b)
    scaled = c * 2.0 ** 48
    ints = np.rint(scaled).astype(np.int64)
    assert np.array_equal(ints.astype(np.float64), scaled), "C * 2^48 is not an integer"
    t = TINY
    with open(os.path.join(HERE, "tiny_w8_m8_k512_n256.txt"), "w") as f:
        f.write("# C * 2^48 of the tiny AG+GEMM workload, written by tests/golden/make_golden.py from the CPU oracle\n")
        f.write("# \"Eliminating Multi-GPU Performance Taxes\" analysis page: C = sum_s A_s . B[sK/W:(s+1)K/W, :]\n")
        f.write(f"# W={t['W']} M={t['M']} K={t['K']} N={t['N']} seed_a={t['seed_a']:#x} seed_b={t['seed_b']:#x}\n")
        f.write(f"# sum of A bit patterns {bits_sum(a)}, sum of B bit patterns {bits_sum(b)}\n")
        for row in ints:
            f.write(" ".join(str(int(v)) for v in row) + "\n")


def write_fd():
    o, lse = fd_inputs()
    out = fdo.combine(o, lse)
    with open(os.path.join(HERE, "fd_w4_h16_d64.txt"), "w") as f:
        f.write("# O of the Flash-Decode global reduction (binary64, float.hex), written by "
                "tests/golden/make_golden.py from the CPU oracle\n")
        f.write("# \"Eliminating Multi-GPU Performance Taxes\" analysis page, Flash Decode global reduction\n")
        f.write(f"# W={FD['W']} H={FD['H']} D={FD['D']} seed={FD['seed']:#x} (synth.fd_partials)\n")
        for row in out:
            f.write(" ".join(float(v).hex() for v in row) + "\n")


if __name__ == "__main__":
    write_tiny()
    write_fd()
    print("wrote", HERE)
