"""Pins for the CPU oracle, against things other than the oracle itself.

The oracle evaluates the AG+GEMM core identity of the "Eliminating Multi-GPU
Performance Taxes" analysis page (symbol table and core equation):
C = sum_s A_s . B[sK/W:(s+1)K/W, :], shards ascending, in binary64.

Pins used here:
  * exhaustive binary16 decoding against numpy's independent implementation;
  * exact integer arithmetic: every input is a multiple of 2^-24, so products
    are multiples of 2^-48 and an int64 matrix product is exact; where every
    running sum stays below 2^5 the binary64 oracle must be *bit-identical*;
  * an unrelated binary64 matrix product (numpy / BLAS) of the unsharded A;
  * W = 1 against a pure-Python sequential loop (bit-identical);
  * shard-order permutation invariance (the page's argument that the
    decomposition is exact, so any order of the shard sum is equally correct);
  * closed forms: one-hot rows, B = 1, A = 0, A supported on one shard;
  * planted mistakes (a transposed operand, a dropped term, a wrong shard to
    B-slice mapping, a sign flip) must each fail at least one pin.
"""
import math
import random

import numpy as np
import pytest

import oracle
import synth


def _f64(bits: np.ndarray) -> np.ndarray:
    return bits.view(np.float16).astype(np.float64)


def _inputs(W, M, K, N, seed=1):
    a = synth.matrix_f16(0xA000 + seed, M, K)
    b = synth.matrix_f16(0xB000 + seed, K, N)
    return a, synth.shards(a, W), b


def _exact_scaled(a_bits, b_bits):
    """Exact C * 2^48 as int64, plus the largest |running sum| * 2^48 along j."""
    ai = np.rint(_f64(a_bits) * 2.0 ** 24).astype(np.int64)
    bi = np.rint(_f64(b_bits) * 2.0 ** 24).astype(np.int64)
    assert np.array_equal(ai.astype(np.float64) * 2.0 ** -24, _f64(a_bits))  # really integers
    assert np.array_equal(bi.astype(np.float64) * 2.0 ** -24, _f64(b_bits))
    c = ai @ bi  # |sum| <= K * 2^48 < 2^63 for K <= 2^14
    return c, ai, bi


# ---------------------------------------------------------------- pins as functions

def pin_direct_product(c, a_bits, b_bits):
    """Unrelated binary64 product of the unsharded A; error bound of recursive summation."""
    A, B = _f64(a_bits), _f64(b_bits)
    ref = A @ B
    bound = 1e-12 * (np.abs(A) @ np.abs(B)) + 1e-300
    return bool((np.abs(c - ref) <= bound).all())


def pin_exact(c, a_bits, b_bits, K):
    cx, _, _ = _exact_scaled(a_bits, b_bits)
    exact = cx.astype(np.float64) * 2.0 ** -48  # exact while |C| < 2^5 (53-bit significand)
    bound = K * K * 2.0 ** -53
    return bool((np.abs(c - exact) <= bound).all())


# ---------------------------------------------------------------- tests

def test_decoder_exhaustive():
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = allbits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_f64(int(b)) for b in allbits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


@pytest.mark.parametrize("W,M,K,N", [(8, 8, 512, 256), (2, 5, 64, 24), (4, 33, 256, 40), (1, 3, 96, 7), (8, 1, 1024, 64)])
def test_against_direct_and_exact(W, M, K, N):
    a, sh, b = _inputs(W, M, K, N, seed=W + M)
    c = oracle.sharded_gemm(sh, b)
    assert pin_direct_product(c, a, b)
    assert pin_exact(c, a, b, K)


def test_tiny_config_bit_exact():
    """Tiny workload (W=8, M=8, K=512, N=256): every running sum stays below 2^5, so the
    binary64 evaluation has no rounding at all and must equal the exact integer result."""
    W, M, K, N = 8, 8, 512, 256
    a, sh, b = _inputs(W, M, K, N, seed=1)
    c = oracle.sharded_gemm(sh, b)
    cx, ai, bi = _exact_scaled(a, b)
    KS = K // W
    # largest running sum inside each shard partial and across shard partials
    prods = ai[:, :, None] * bi[None, :, :]  # M x K x N, int64 exact
    run = 0
    for s in range(W):
        cs = np.cumsum(prods[:, s * KS:(s + 1) * KS, :], axis=1)
        run = max(run, int(np.abs(cs).max()))
    parts = np.stack([prods[:, s * KS:(s + 1) * KS, :].sum(axis=1) for s in range(W)])
    run = max(run, int(np.abs(np.cumsum(parts, axis=0)).max()))
    assert run < 2 ** 53  # every intermediate is exactly representable
    assert np.array_equal(c, cx.astype(np.float64) * 2.0 ** -48)


def test_w1_equals_sequential_python_loop():
    M, K, N = 3, 40, 5
    a, sh, b = _inputs(1, M, K, N, seed=7)
    c = oracle.sharded_gemm(sh, b)
    A, B = _f64(a), _f64(b)
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for j in range(K):
                acc += float(A[m, j]) * float(B[j, n])
            assert c[m, n] == acc


def test_shard_order_permutation_invariance():
    W, M, K, N = 8, 6, 2048, 48
    _, sh, b = _inputs(W, M, K, N, seed=3)
    c = oracle.sharded_gemm(sh, b)
    parts = [oracle.shard_partial(sh, b, s) for s in range(W)]
    # ascending order reproduces the oracle bit for bit
    acc = np.zeros_like(c)
    for p in parts:
        acc = acc + p
    assert np.array_equal(acc, c)
    rng = random.Random(5)
    scale = np.abs(np.stack(parts)).sum(axis=0)
    for _ in range(20):
        order = list(range(W))
        rng.shuffle(order)
        acc = np.zeros_like(c)
        for s in order:
            acc = acc + parts[s]
        assert (np.abs(acc - c) <= W * 2.0 ** -52 * scale + 1e-300).all()


def test_partials_pin_shard_to_b_slice_mapping():
    W, M, K, N = 4, 5, 256, 16
    a, sh, b = _inputs(W, M, K, N, seed=11)
    KS = K // W
    cx, ai, bi = _exact_scaled(a, b)
    for s in range(W):
        p = oracle.shard_partial(sh, b, s)
        ex = (ai[:, s * KS:(s + 1) * KS] @ bi[s * KS:(s + 1) * KS, :]).astype(np.float64) * 2.0 ** -48
        assert np.array_equal(p, ex)


def test_closed_forms():
    W, M, K, N = 4, 6, 256, 32
    _, sh, b = _inputs(W, M, K, N, seed=13)
    KS = K // W
    one = np.uint16(0x3C00)
    # one-hot rows: row m selects global column k_m -> C row equals B row k_m exactly
    picks = [0, KS - 1, KS, 2 * KS + 5, K - 1, 3 * KS]
    a = np.zeros((M, K), dtype=np.uint16)
    for m, k in enumerate(picks):
        a[m, k] = one
    c = oracle.sharded_gemm(synth.shards(a, W), b)
    for m, k in enumerate(picks):
        assert np.array_equal(c[m], _f64(b[k]))
    # B = 1 -> C[m, :] = sum_k A[m, k] (exact: fp16 inputs, binary64 sum of <= 2^10 terms)
    a2, sh2, _ = _inputs(W, M, K, N, seed=17)
    ones = np.full((K, N), one, dtype=np.uint16)
    c = oracle.sharded_gemm(sh2, ones)
    rows = [math.fsum(_f64(a2[m]).tolist()) for m in range(M)]
    for m in range(M):
        assert (c[m] == rows[m]).all()
    # A = 0 -> C = 0
    z = [np.zeros((M, KS), dtype=np.uint16) for _ in range(W)]
    assert not oracle.sharded_gemm(z, b).any()
    # A supported on shard 2 only: C equals P_2, and rows of B outside shard 2 do not matter
    only = [np.zeros((M, KS), dtype=np.uint16) for _ in range(W)]
    only[2] = sh2[2]
    c = oracle.sharded_gemm(only, b)
    b_mut = b.copy()
    b_mut[:2 * KS] = synth.matrix_f16(0xBEEF, 2 * KS, N)
    b_mut[3 * KS:] = synth.matrix_f16(0xBEEE, K - 3 * KS, N)
    assert np.array_equal(c, oracle.sharded_gemm(only, b_mut))
    assert np.array_equal(c, oracle.shard_partial(only, b, 2))


def test_entries_match_full_evaluation():
    W, M, K, N = 8, 17, 512, 72
    _, sh, b = _inputs(W, M, K, N, seed=19)
    c = oracle.sharded_gemm(sh, b)
    rows = np.array([0, 16, 5, 9, 16, 3])
    cols = np.array([0, 71, 33, 64, 0, 8])
    assert np.array_equal(oracle.sharded_gemm_entries(sh, b, rows, cols), c[rows, cols])
    with pytest.raises(RuntimeError):
        oracle.sharded_gemm_entries(sh, b, np.array([17]), np.array([0]))


def test_thread_count_does_not_change_result():
    W, M, K, N = 8, 13, 1024, 40
    _, sh, b = _inputs(W, M, K, N, seed=23)
    assert np.array_equal(oracle.sharded_gemm(sh, b, nthreads=1), oracle.sharded_gemm(sh, b, nthreads=7))


def test_empty_m_and_bad_shapes():
    b = synth.matrix_f16(1, 64, 8)
    sh = [np.zeros((0, 16), dtype=np.uint16) for _ in range(4)]
    assert oracle.sharded_gemm(sh, b).shape == (0, 8)
    with pytest.raises(ValueError):
        oracle.sharded_gemm([np.zeros((2, 16), dtype=np.uint16)] * 4, synth.matrix_f16(1, 60, 8))


# ---------------------------------------------------------------- the pins catch planted mistakes

def _planted_variants(sh, b):
    """Plausible mistakes, built on the CPU from the oracle's own partials."""
    W = len(sh)
    KS = sh[0].shape[1]
    A = np.concatenate([_f64(s) for s in sh], axis=1)
    B = _f64(b)
    out = {}
    # wrong shard -> B slice mapping (s uses the rows of shard s+1)
    out["shifted_b_slice"] = sum(_f64(sh[s]) @ B[((s + 1) % W) * KS:((s + 1) % W + 1) * KS] for s in range(W))
    # dropped last term of each shard's inner sum
    out["dropped_term"] = sum(_f64(sh[s])[:, :-1] @ B[s * KS:(s + 1) * KS - 1] for s in range(W))
    # dropped shard
    out["dropped_shard"] = sum(_f64(sh[s]) @ B[s * KS:(s + 1) * KS] for s in range(W - 1))
    # sign flip on one shard
    out["sign_flip"] = sum((-1 if s == 1 else 1) * (_f64(sh[s]) @ B[s * KS:(s + 1) * KS]) for s in range(W))
    # transposed B rows inside a shard (reversed j order of B only)
    out["reversed_rows"] = sum(_f64(sh[s]) @ B[s * KS:(s + 1) * KS][::-1] for s in range(W))
    # A columns taken in the wrong order across shards
    out["shard_swap_a"] = sum(_f64(sh[(s + 1) % W]) @ B[s * KS:(s + 1) * KS] for s in range(W))
    return out


def test_pins_reject_planted_mistakes():
    W, M, K, N = 4, 6, 256, 24
    a, sh, b = _inputs(W, M, K, N, seed=29)
    good = oracle.sharded_gemm(sh, b)
    assert pin_direct_product(good, a, b) and pin_exact(good, a, b, K)
    for name, bad in _planted_variants(sh, b).items():
        assert not pin_direct_product(bad, a, b), name
        assert not pin_exact(bad, a, b, K), name
