"""Readers of the stored expected values in tests/golden/ (written by
tests/golden/make_golden.py from the CPU oracle)."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        lines = f.read().splitlines()
    head = [ln for ln in lines if ln.startswith("#")]
    body = [ln.split() for ln in lines if ln and not ln.startswith("#")]
    return head, body


def tiny():
    """(header lines, C * 2^48 as an int64 M x N array) of the tiny AG+GEMM workload."""
    head, body = _rows("tiny_w8_m8_k512_n256.txt")
    return head, np.array([[int(v) for v in r] for r in body], dtype=np.int64)


def tiny_c():
    """The tiny workload's C as binary64 (exact: |C| < 2^5, multiples of 2^-48)."""
    return tiny()[1].astype(np.float64) * 2.0 ** -48


def fd():
    """O (H x D, binary64) of the stored Flash-Decode combine case."""
    _, body = _rows("fd_w4_h16_d64.txt")
    return np.array([[float.fromhex(v) for v in r] for r in body], dtype=np.float64)
