"""Pins for the seeded input generator (shared by the oracle and the GPU path).

The generator is checked against things other than itself: the published
first output of splitmix64, an independent numpy evaluation of the same
counter hash, and numpy's own binary64 -> binary16 rounding.
"""
import numpy as np
import pytest

import synth

MASK = (1 << 64) - 1


def _splitmix64_numpy(x: np.ndarray) -> np.ndarray:
    # Independent vectorised evaluation of the splitmix64 finaliser (uint64 wraps mod 2^64).
    with np.errstate(over="ignore"):
        z = x + np.uint64(0x9E3779B97F4A7C15)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
        return z ^ (z >> np.uint64(31))


def test_splitmix64_published_vector():
    # First outputs of the splitmix64 generator started from state 0 (Vigna's reference
    # generator adds the golden gamma before mixing, which is exactly our hash of 0, gamma, 2*gamma).
    g = 0x9E3779B97F4A7C15
    assert synth.splitmix64(0) == 0xE220A8397B1DCDAF
    assert synth.splitmix64(g) == 0x6E789E6AA1B965F4
    assert synth.splitmix64((2 * g) & MASK) == 0x06C45D188009454F


def test_splitmix64_matches_numpy():
    xs = np.arange(0, 5000, dtype=np.uint64) * np.uint64(0x1234567) ^ np.uint64(0xA003)
    ref = _splitmix64_numpy(xs)
    got = np.array([synth.splitmix64(int(x)) for x in xs], dtype=np.uint64)
    assert np.array_equal(ref, got)


def test_fill_equals_numpy_rounding():
    seed, n = 0xB002, 1 << 20
    bits = synth.fill_f16(seed, n)
    idx = np.arange(n, dtype=np.uint64)
    u = _splitmix64_numpy(np.uint64(seed) ^ idx) >> np.uint64(40)
    x = u.astype(np.float64) * 2.0 ** -23 - 1.0
    ref = x.astype(np.float16).view(np.uint16)  # numpy rounds to nearest even
    assert np.array_equal(bits, ref)
    vals = bits.view(np.float16).astype(np.float64)
    assert vals.min() >= -1.0 and vals.max() <= 1.0
    assert abs(vals.mean()) < 0.01 and abs(vals.var() - 1.0 / 3.0) < 0.01


def test_f16_encoder_edge_cases():
    cases = [0.0, -0.0, 1.0, -1.0, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -14, 65504.0, 65520.0,
             1.0 - 2.0 ** -12, 1.0 - 2.0 ** -23, 0.1, -0.3333333333, 2.0 ** -14 - 2.0 ** -25, 1e-30, 7e4]
    for x in cases:
        assert synth.f64_to_f16_bits(x) == int(np.float64(x).astype(np.float16).view(np.uint16)), x


def test_slices_are_consistent_and_deterministic():
    full = synth.fill_f16(0xA004, 10000)
    assert np.array_equal(full[1234:5678], synth.fill_f16(0xA004, 5678 - 1234, start=1234))
    assert np.array_equal(full, synth.fill_f16(0xA004, 10000))
    assert not np.array_equal(full, synth.fill_f16(0xA005, 10000))


def test_shards_are_column_slices():
    a = synth.matrix_f16(0xA001, 8, 512)
    sh = synth.shards(a, 8)
    assert len(sh) == 8 and all(s.shape == (8, 64) for s in sh)
    assert np.array_equal(np.concatenate(sh, axis=1), a)
    with pytest.raises(ValueError):
        synth.shards(a, 7)


def test_schedule_is_permutation_with_cumulative_delays():
    order, offs = synth.schedule(0x5005, 32, 20000)
    assert sorted(order.tolist()) == list(range(32))
    d = np.diff(np.concatenate([[0], offs]))
    assert (d >= 0).all() and (d <= 20000).all()
    # expected span ~ 32 * 10 us
    assert 150_000 < offs[-1] < 500_000
    o2, f2 = synth.schedule(0x5005, 32, 20000)
    assert np.array_equal(order, o2) and np.array_equal(offs, f2)
    o0, f0 = synth.schedule(0x5005, 32, 0)
    assert (f0 == 0).all() and np.array_equal(o0, order)


@pytest.mark.parametrize("lo,hi", [(-1.0, 1.0), (8.0, 16.0)])
def test_fill_f32_recipe(lo, hi):
    """fp32 stream: lo + (hi - lo) * u * 2^-24 in binary64, rounded to binary32 by numpy."""
    seed, n, start = 0x7003, 1 << 16, 12345
    got = synth.fill_f32(seed, n, lo, hi, start=start)
    idx = np.arange(start, start + n, dtype=np.uint64)
    u = _splitmix64_numpy(np.uint64(seed) ^ idx) >> np.uint64(40)
    ref = (lo + (hi - lo) * (u.astype(np.float64) * 2.0 ** -24)).astype(np.float32)
    assert np.array_equal(got, ref)
    assert got.min() >= lo and got.max() < hi
    if (lo, hi) == (-1.0, 1.0):
        # every value is a multiple of 2^-23 in [-1, 1): exact in binary32
        assert np.array_equal(got.astype(np.float64), lo + (hi - lo) * (u.astype(np.float64) * 2.0 ** -24))


def test_fd_partials_streams():
    o, lse = synth.fd_partials(0x7100, 3, 4, 8)
    assert len(o) == 3 and len(lse) == 3
    assert o[1].shape == (4, 8) and lse[2].shape == (4,)
    assert np.array_equal(o[1].ravel(), synth.fill_f32(0x7102, 32))
    assert np.array_equal(lse[2], synth.fill_f32(0x7105, 4, 8.0, 16.0))
