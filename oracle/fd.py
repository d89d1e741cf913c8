"""CPU oracle for the Flash-Decode online-softmax combine (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module; the product path never does. It is plain
numpy in binary64 and shares nothing with the GPU path.

"Eliminating Multi-GPU Performance Taxes" analysis page, Flash Decode global
reduction and correctness check #5: the final attention output of one query
is the online-softmax combine of the W per-rank partial outputs, and the
combine may take the partials in any order. A partial is read here as the
normalised attention output of rank s over its own KV shard, o_s (H x D),
with the log-sum-exp of its scores, lse_s (H); for each head h

    O[h] = sum_s exp(lse_s[h] - m) * o_s[h] / sum_s exp(lse_s[h] - m),
    m = max_s lse_s[h].

An online combine (running maximum, rescaled running sums) reaches this
value up to rounding, so the oracle is the weighted average written out, with
the partials visited in ascending s. ``attention`` and ``attention_partial``
exist only to pin it: the combine of the partials of any split of a KV cache
must equal softmax attention over the whole cache.
"""
from __future__ import annotations

import numpy as np


def combine(o_parts, lse_parts) -> np.ndarray:
    """O (H x D, binary64) from W partial outputs (H x D) and log-sum-exps (H)."""
    W = len(o_parts)
    if W < 1 or len(lse_parts) != W:
        raise ValueError("need W >= 1 partial outputs and as many log-sum-exp vectors")
    o = [np.asarray(x, dtype=np.float64) for x in o_parts]
    lse = [np.asarray(x, dtype=np.float64) for x in lse_parts]
    H, D = o[0].shape
    for s in range(W):
        if o[s].shape != (H, D) or lse[s].shape != (H,):
            raise ValueError("partial shapes differ")
    m = lse[0].copy()
    for s in range(1, W):
        m = np.maximum(m, lse[s])
    num = np.zeros((H, D))
    den = np.zeros(H)
    for s in range(W):
        w = np.exp(lse[s] - m)
        num += w[:, None] * o[s]
        den += w
    return num / den[:, None]


def attention(q, K, V, scale: float) -> np.ndarray:
    """Softmax attention of one query per head over a whole KV cache (binary64).
    q: H x D; K, V: L x H x D. Returns H x D."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    L, H, D = K.shape
    out = np.empty((H, D))
    for h in range(H):
        s = scale * (K[:, h, :] @ q[h])           # L scores
        p = np.exp(s - s.max())
        p /= p.sum()
        out[h] = p @ V[:, h, :]
    return out


def attention_partial(q, K, V, scale: float):
    """One rank's partial over its KV shard: (o, lse), o normalised (H x D), lse (H)."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    L, H, D = K.shape
    if L < 1:
        raise ValueError("a partial needs at least one key")
    o = np.empty((H, D))
    lse = np.empty(H)
    for h in range(H):
        s = scale * (K[:, h, :] @ q[h])
        mx = s.max()
        e = np.exp(s - mx)
        o[h] = (e @ V[:, h, :]) / e.sum()
        lse[h] = mx + np.log(e.sum())
    return o, lse


def tolerance(out_dtype: str) -> float:
    """Bound on |O_gpu - O_oracle| for partial outputs in [-1, 1] and W <= 16.

    The GPU combines in binary32: each weight exp(lse_s - m) carries a few ulp
    of relative error (the exponent argument is rounded, then exp itself),
    and the weighted sum of at most 16 terms adds one rounding per term, so
    the error stays below 16 * 2^-19 * max|o| = 3.1e-5. A binary16 output adds
    half an ulp at |O| < 1 (2^-12 = 2.4e-4)."""
    base = 16 * 2.0 ** -19
    if out_dtype == "f16":
        return base + 2.0 ** -12
    if out_dtype == "f32":
        return base
    raise ValueError(out_dtype)
