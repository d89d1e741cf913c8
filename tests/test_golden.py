"""Stored expected values (tests/golden/) against the generator, brute force and
the oracle.

tiny_w8_m8_k512_n256.txt holds C * 2^48 of the tiny AG+GEMM workload ("Eliminating
Multi-GPU Performance Taxes" analysis page, core identity). Its integers are checked
against an exact int64 product of the unsharded inputs, which shares nothing with
the oracle, and the oracle must reproduce them bit for bit. fd_w4_h16_d64.txt holds
the Flash-Decode global reduction of seeded partials (same page); the oracle must
reproduce it bit for bit, and every output must lie between the smallest and the
largest partial (the combine is a convex combination of the ranks' outputs).
"""
import re

import numpy as np

import oracle
import synth
from oracle import fd as fdo
from tests import golden_io


def _tiny_inputs():
    head, _ = golden_io.tiny()
    meta = dict(re.findall(r"(\w+)=(0x[0-9a-f]+|\d+)", " ".join(head)))
    W, M, K, N = (int(meta[k]) for k in ("W", "M", "K", "N"))
    a = synth.matrix_f16(int(meta["seed_a"], 16), M, K)
    b = synth.matrix_f16(int(meta["seed_b"], 16), K, N)
    return head, W, a, b


def test_tiny_golden_inputs_regenerate():
    head, W, a, b = _tiny_inputs()
    sums = [int(x) for x in re.findall(r"bit patterns (\d+)", " ".join(head))]
    assert sums == [int(a.astype(np.uint64).sum()), int(b.astype(np.uint64).sum())]


def test_tiny_golden_is_the_exact_product():
    _, W, a, b = _tiny_inputs()
    ai = np.rint(a.view(np.float16).astype(np.float64) * 2.0 ** 24).astype(np.int64)
    bi = np.rint(b.view(np.float16).astype(np.float64) * 2.0 ** 24).astype(np.int64)
    _, c48 = golden_io.tiny()
    assert np.array_equal(ai @ bi, c48)


def test_oracle_reproduces_tiny_golden():
    _, W, a, b = _tiny_inputs()
    assert np.array_equal(oracle.sharded_gemm(synth.shards(a, W), b), golden_io.tiny_c())


def test_oracle_reproduces_fd_golden():
    o, lse = synth.fd_partials(0x7A00, 4, 16, 64)
    ref = golden_io.fd()
    assert ref.shape == (16, 64)
    assert np.array_equal(fdo.combine(o, lse), ref)
    lo = np.min(np.stack(o), axis=0).astype(np.float64)
    hi = np.max(np.stack(o), axis=0).astype(np.float64)
    assert ((ref >= lo) & (ref <= hi)).all()
