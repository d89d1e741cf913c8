"""Shapes at the size limits the library accepts (agemm_create: N <= 2^24 and
K <= 2^22, which keep every lane's 16-byte load offset in 32 bits), every
entry of C against the oracle.

- N = 2^24 columns with one shard of 64 (B is 2 GiB): the small-M kernel at
  M = 1 (32,768 column blocks on a persistent grid), and the MFMA kernel at
  M = 2 (131,072 tiles of 128 columns, a single k-step each, so the direct-load
  cursor crosses into a new tile at every step; nontemporal B).
- K = 2^22 with W = 8 (a shard of 524,288 columns, flag tiles of 65,536): the
  MFMA kernel under the stream-K split on ragged rows and columns, and at
  M = 1, where the small-M kernel's LDS cannot hold a K-range and the MFMA
  kernel takes the shape.

Uniform[-1, 1] inputs, max|err| <= 1e-3 * sqrt(K); the fused (producer
releasing tiles out of order while the consumer runs), BSP and Pull paths run
the same kernel and must agree bit for bit.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

CASES = {
    # name: (W, M, K, N, C dtype, expected consumer)
    "n_limit_small_m": (1, 1, 64, 1 << 24, "f16", dict(kind="small_m")),
    "n_limit_mfma": (1, 2, 64, 1 << 24, "f16", dict(kind="mfma", tile_config=1, tiles=131072, split=0)),
    "k_limit_split": (8, 3, 1 << 22, 136, "f32", dict(kind="mfma", tile_config=1, tiles=2, split=1)),
    "k_limit_m1": (8, 1, 1 << 22, 136, "f32", dict(kind="mfma", tile_config=1, tiles=2, split=1)),
}

_weights = {}


def _weight(W, K, N):
    """B (host bits and device copy), one per shape: the cases of one limit share it."""
    key = (W, K, N)
    if key not in _weights:
        _weights.clear()
        b = synth.matrix_f16(0xE600 + W, K, N)
        _weights[key] = (b, gu.to_dev(b))
    return _weights[key]


@pytest.mark.parametrize("name", list(CASES))
def test_size_limits_every_entry(name):
    import torch
    from shard_decomposed_gemm_amd import Context
    W, M, K, N, c_dtype, expect = CASES[name]
    print(f"[limits] {name} W={W} M={M} K={K} N={N} C={c_dtype}", flush=True)
    a = synth.matrix_f16(0xE500 + M, M, K)
    b, B = _weight(W, K, N)
    sh = synth.shards(a, W)
    ref = oracle.sharded_gemm(sh, b)
    dsh = [gu.to_dev(s) for s in sh]
    ctx = Context(W, M, K, N, c_dtype=c_dtype)
    info = ctx.consumer_info()
    for k, v in expect.items():
        assert info[k] == v, (k, info)
    sched = synth.schedule(0xE700 + M, ctx.t, 2_000)
    outs = {}
    sp, sc = ctx.streams()
    C = gu.empty_c(M, N, c_dtype)
    ctx.produce(dsh, schedule=sched, stream=sp)
    ctx.run_fused(B, C, stream=sc)
    outs["fused"] = C
    C = gu.empty_c(M, N, c_dtype)
    ctx.run_bsp(dsh, B, C, schedule=sched, host_sync=True)
    outs["bsp"] = C
    C = gu.empty_c(M, N, c_dtype)
    ctx.run_pull(dsh, B, C)
    outs["pull"] = C
    torch.cuda.synchronize()
    ctx.check()
    iv = (lambda x: x.view(torch.int16)) if c_dtype == "f16" else (lambda x: x.view(torch.int32))
    assert torch.equal(iv(outs["fused"]), iv(outs["bsp"]))
    assert torch.equal(iv(outs["fused"]), iv(outs["pull"]))
    got = gu.c_to_f64(outs["fused"])
    assert np.isfinite(got).all()
    err = np.abs(got - ref).max()
    assert err <= oracle.tolerance(K), (name, err)
    ctx.close()
    if name == list(CASES)[-1]:
        _weights.clear()
