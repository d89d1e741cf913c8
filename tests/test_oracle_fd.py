"""Pins of the Flash-Decode combine oracle (CPU only).

Each check ties ``oracle.fd.combine`` to something other than itself: softmax
attention over a whole KV cache (the combine of the partials of any split
must reproduce it), the order freedom of correctness check #5 of the
"Eliminating Multi-GPU Performance Taxes" analysis page, and closed-form
cases (one partial, equal statistics, a dominant partial, a hand example,
a common shift of all statistics).
"""
import math

import numpy as np
import pytest

from oracle import fd


def _qkv(seed, L, H, D):
    rng = np.random.default_rng(seed)
    q = rng.uniform(-1, 1, (H, D))
    K = rng.uniform(-1, 1, (L, H, D))
    V = rng.uniform(-1, 1, (L, H, D))
    return q, K, V


@pytest.mark.parametrize("cuts", [[16, 32, 48], [1, 2, 63], [5], [7, 8, 9, 30, 31, 40, 50]])
def test_combine_of_split_equals_full_attention(cuts):
    """Split a 64-key cache at arbitrary points (uneven shards, one-key shards);
    combining the shards' partials gives softmax attention over the whole cache."""
    L, H, D = 64, 4, 8
    q, K, V = _qkv(11, L, H, D)
    scale = 1.0 / math.sqrt(D) * 3.0  # sharpen the softmax so the weights differ widely
    bounds = [0] + list(cuts) + [L]
    parts = [fd.attention_partial(q, K[a:b], V[a:b], scale) for a, b in zip(bounds[:-1], bounds[1:])]
    got = fd.combine([p[0] for p in parts], [p[1] for p in parts])
    ref = fd.attention(q, K, V, scale)
    assert np.abs(got - ref).max() < 1e-13


def test_combine_order_free():
    """Check #5: any order of the partials gives the same output (up to rounding)."""
    H, D, W = 6, 16, 8
    rng = np.random.default_rng(3)
    o = [rng.uniform(-1, 1, (H, D)) for _ in range(W)]
    lse = [rng.uniform(8, 16, H) for _ in range(W)]
    ref = fd.combine(o, lse)
    for perm in (list(range(W))[::-1], [3, 1, 7, 0, 6, 2, 5, 4]):
        got = fd.combine([o[i] for i in perm], [lse[i] for i in perm])
        assert np.abs(got - ref).max() < 1e-15


def test_single_partial_is_identity():
    o = np.random.default_rng(4).uniform(-1, 1, (3, 5))
    lse = np.array([1.0, -7.0, 300.0])
    assert np.array_equal(fd.combine([o], [lse]), o)


def test_equal_statistics_give_the_mean():
    rng = np.random.default_rng(5)
    o = [rng.uniform(-1, 1, (2, 4)) for _ in range(4)]
    lse = [np.full(2, 9.25) for _ in range(4)]
    assert np.abs(fd.combine(o, lse) - sum(o) / 4).max() < 1e-15


def test_dominant_partial_without_overflow():
    """Statistics a thousand apart: exp(lse) would overflow binary64, the combine must not;
    the dominant partial's weight is 1 to within exp(-1000)."""
    rng = np.random.default_rng(6)
    o = [rng.uniform(-1, 1, (2, 3)) for _ in range(3)]
    lse = [np.array([1000.0, -5.0]), np.array([0.0, 995.0]), np.array([-1.0, -6.0])]
    got = fd.combine(o, lse)
    assert np.isfinite(got).all()
    assert np.array_equal(got[0], o[0][0])
    assert np.array_equal(got[1], o[1][1])


def test_hand_example():
    """Statistics 0 and ln 3 weigh the partials 1/4 and 3/4: (4 + 3*8) / 4 = 7."""
    got = fd.combine([np.array([[4.0]]), np.array([[8.0]])], [np.array([0.0]), np.array([math.log(3.0)])])
    assert abs(got[0, 0] - 7.0) < 1e-15


def test_common_shift_of_statistics_changes_nothing():
    rng = np.random.default_rng(7)
    o = [rng.uniform(-1, 1, (3, 4)) for _ in range(5)]
    lse = [rng.uniform(8, 16, 3) for _ in range(5)]
    ref = fd.combine(o, lse)
    for c in (-40.0, 123.5):
        assert np.abs(fd.combine(o, [x + c for x in lse]) - ref).max() < 1e-14


def test_partial_of_one_key():
    """A shard with one key: its output is that key's value row, its statistic the score."""
    q, K, V = _qkv(8, 1, 2, 4)
    o, lse = fd.attention_partial(q, K, V, 0.5)
    assert np.allclose(o, V[0])
    assert np.allclose(lse, 0.5 * np.einsum("hd,hd->h", K[0], q))


def test_tolerance_values():
    assert fd.tolerance("f32") == pytest.approx(3.0517578125e-05)
    assert fd.tolerance("f16") == pytest.approx(3.0517578125e-05 + 2.44140625e-04)
    with pytest.raises(ValueError):
        fd.tolerance("bf16")
