"""Arrival-order consumption of the flag tiles on the GPU.

The AG+GEMM core identity ("Eliminating Multi-GPU Performance Taxes"
analysis page) writes C as a plain sum of per-shard partial products, so the
shards may be taken in any order; the consumer in arrival order takes, per
output tile, the raised flag tiles first. Checks: exact inputs give the
oracle bit for bit in any order; random inputs stay within the tolerance; a
poisoned inbox is never read early; with every flag up at launch the result
equals the shard-order one bit for bit; a late first shard costs the
arrival-order consumer only the tail of the work; and with 64 flag tiles the
order never reaches past the last tile (a sign-extended 64-bit record of
raised flags once made tiles 32..63 look raised).
"""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _whole_tiles(monkeypatch):
    """Arrival order runs on whole tiles; the shard-order contexts these tests compare
    with are kept on whole tiles too (the stream-K split groups the sum differently)."""
    monkeypatch.setenv("AGEMM_SPLIT", "0")


def _ctx(W, M, K, N, c_dtype="f32", order="arrival"):
    from shard_decomposed_gemm_amd import Context
    ctx = Context(W, M, K, N, c_dtype=c_dtype)
    ctx.set_order(order)
    return ctx


def _poison(ctx, W, M, K):
    """Fill both inboxes (epochs alternate between them) with fp16 NaN."""
    import torch
    nan = [torch.full((M, K // W), float("nan"), dtype=torch.float16, device=gu.dev()) for _ in range(W)]
    ctx.produce(nan)
    ctx.produce(nan)
    torch.cuda.synchronize()


def _fused_concurrent(ctx, dsh, B, C, schedule):
    import torch
    sp, sc = ctx.streams()
    ctx.produce(dsh, schedule=schedule, stream=sp)
    ctx.run_fused(B, C, stream=sc)
    torch.cuda.synchronize()
    ctx.check()


@pytest.mark.parametrize("tile_config", [0, 1, 2])
@pytest.mark.parametrize("W,M,K,N", [(8, 300, 2048, 1032), (4, 520, 1024, 264), (16, 257, 1024, 264)])
def test_arrival_exact_inputs_bitwise(tile_config, W, M, K, N, monkeypatch):
    """Exact inputs (every partial sum exact in fp32): whatever order the tiles arrive
    and are taken in, C equals the oracle bit for bit. Released out of order with up to
    20 us between tiles into a poisoned inbox, on every tile configuration."""
    monkeypatch.setenv("AGEMM_TILE_CONFIG", str(tile_config))
    a = gu.coarse_bits(0xF000 + M, M, K)
    b = gu.coarse_bits(0xF100 + N, K, N)
    sh = synth.shards(a, W)
    ref = oracle.sharded_gemm(sh, b)
    dsh = [gu.to_dev(s) for s in sh]
    B = gu.to_dev(b)
    ctx = _ctx(W, M, K, N)
    _poison(ctx, W, M, K)
    for rep in range(2):
        order, offs = synth.schedule(0xF200 + 4 * tile_config + rep, ctx.t, 20_000)
        C = gu.empty_c(M, N, "f32")
        _fused_concurrent(ctx, dsh, B, C, (order, offs))
        assert np.array_equal(C.cpu().numpy().astype(np.float64), ref), (tile_config, rep)


@pytest.mark.parametrize("W,M,K,N", [(8, 96, 2048, 1024), (8, 512, 2048, 1024), (8, 300, 4096, 2056)])
@pytest.mark.parametrize("c_dtype", ["f16", "f32"])
def test_arrival_random_within_tolerance(W, M, K, N, c_dtype):
    """Random inputs, poisoned inbox, seeded out-of-order release: within 1e-3 * sqrt(K)
    of the oracle (only the fp32 summation order differs from shard order)."""
    a, sh, b, dsh, B = gu.random_problem(W, M, K, N, seed=M + 3)
    ref = oracle.sharded_gemm(sh, b)
    ctx = _ctx(W, M, K, N, c_dtype)
    _poison(ctx, W, M, K)
    order, offs = synth.schedule(0xF300 + M, ctx.t, 40_000)
    C = gu.empty_c(M, N, c_dtype)
    _fused_concurrent(ctx, dsh, B, C, (order, offs))
    got = gu.c_to_f64(C)
    assert np.isfinite(got).all()
    assert np.abs(got - ref).max() <= oracle.tolerance(K)


def test_arrival_flags_preset_equals_shard_order():
    """Every flag raised before the launch: the arrival-order consumer runs in shard
    order, so its C equals the shard-order consumer's bit for bit (random inputs)."""
    import torch
    W, M, K, N = 8, 300, 2048, 1032
    a, sh, b, dsh, B = gu.random_problem(W, M, K, N, seed=5)
    outs = []
    for order in ("shard", "arrival"):
        ctx = _ctx(W, M, K, N, "f32", order=order)
        ctx.produce(dsh)
        torch.cuda.synchronize()
        C = gu.empty_c(M, N, "f32")
        ctx.run_fused(B, C)
        torch.cuda.synchronize()
        ctx.check()
        outs.append(C.cpu().numpy())
    assert np.array_equal(outs[0], outs[1])
    assert np.abs(outs[1].astype(np.float64) - oracle.sharded_gemm(sh, b)).max() <= oracle.tolerance(K)


def test_arrival_epochs_switch_order():
    """Shard and arrival order alternate over epochs on one context (both inboxes in
    use, out-of-order releases): every epoch matches its own data set."""
    import torch
    W, M, K, N = 8, 256, 2048, 1024
    probs = [gu.random_problem(W, M, K, N, seed=s) for s in (111, 112, 113)]
    refs = [oracle.sharded_gemm(p[1], p[2]) for p in probs]
    ctx = _ctx(W, M, K, N)
    sp, sc = ctx.streams()
    outs = []
    for e in range(6):
        p = probs[e % 3]
        ctx.set_order("arrival" if e % 2 == 0 else "shard")
        order, offs = synth.schedule(0xF400 + e, ctx.t, 10_000)
        C = gu.empty_c(M, N, "f32")
        ctx.produce(p[3], schedule=(order, offs), stream=sp)
        ctx.run_fused(p[4], C, stream=sc)
        outs.append(C)
    torch.cuda.synchronize()
    ctx.check()
    for e, C in enumerate(outs):
        assert np.abs(gu.c_to_f64(C) - refs[e % 3]).max() <= oracle.tolerance(K), e


def test_arrival_late_first_shard_costs_only_the_tail():
    """Shard 0's first k-tile is released last, 3 ms after the others. In shard order
    every workgroup waits for it before any work; in arrival order the workgroups do
    the other 31 k-tiles meanwhile, so the consumer kernel ends well before the
    shard-order one (by most of the GEMM's own duration). Both results are checked on
    sampled rows against the oracle."""
    import torch
    W, M, K, N = 8, 1024, 8192, 8192
    a, sh, b, dsh, B = gu.random_problem(W, M, K, N, seed=121)
    rows = np.arange(0, M, 67)
    ref = oracle.sharded_gemm([s[rows] for s in sh], b)
    dur = {}
    for order in ("shard", "arrival"):
        ctx = _ctx(W, M, K, N, "f32", order=order)
        T = ctx.t
        rel = np.concatenate([np.arange(1, T), [0]]).astype(np.int32)
        offs = np.zeros(T, dtype=np.int64)
        offs[-1] = 3_000_000
        # one concurrent run to warm up, then the timed one
        times = []
        for rep in range(2):
            C = gu.empty_c(M, N, "f32")
            ctx.timing_begin(1)
            _fused_concurrent(ctx, dsh, B, C, (rel, offs))
            times.append(ctx.timing_end()[0])
            got = gu.c_to_f64(C)[rows]
            assert np.abs(got - ref).max() <= oracle.tolerance(K), (order, rep)
        dur[order] = times[-1]
    pull_ctx = _ctx(W, M, K, N, "f32", order="shard")
    C = gu.empty_c(M, N, "f32")
    pull_ctx.timing_begin(2)
    pull_ctx.run_pull(dsh, B, C)
    pull_ctx.run_pull(dsh, B, C)
    torch.cuda.synchronize()
    gemm_us = pull_ctx.timing_end()[-1]
    print(f"consumer kernel: shard order {dur['shard']:.0f} us, arrival order {dur['arrival']:.0f} us, "
          f"GEMM alone {gemm_us:.0f} us")
    if dur["shard"] < 2_500:
        pytest.skip("producer and consumer did not overlap (the consumer never waited)")
    assert dur["arrival"] < dur["shard"] - 0.5 * gemm_us


def test_arrival_sixty_four_flags_late_high_tiles():
    """T = 64: tiles 0..31 (tile 31 first) released at once, tiles 32..63 two milliseconds
    later, into poisoned inboxes. The arrival order takes the raised tiles first and must
    then wait for each of 32..63, never take a tile it has not seen raised, and never
    pick an id at or beyond T."""
    import torch
    W, M, K, N, bkf = 8, 300, 8192, 1000, 128
    a, sh, b, dsh, B = gu.random_problem(W, M, K, N, seed=49)
    ref = oracle.sharded_gemm(sh, b)
    from shard_decomposed_gemm_amd import Context
    ctx = Context(W, M, K, N, c_dtype="f32", flag_ktile=bkf)
    ctx.set_order("arrival")
    assert ctx.t == 64
    order = np.array([31] + list(range(31)) + list(range(32, 64)), dtype=np.int32)
    offs = np.array([0] * 32 + [2_000_000 + 1_000 * i for i in range(32)], dtype=np.int64)
    for _ in range(3):
        _poison(ctx, W, M, K)
        C = gu.empty_c(M, N, "f32")
        _fused_concurrent(ctx, dsh, B, C, (order, offs))
        got = gu.c_to_f64(C)
        assert np.isfinite(got).all()
        assert np.abs(got - ref).max() <= oracle.tolerance(K)
    ctx.close()
