"""The MFMA consumer's stream-K split on the GPU.

With fewer output tiles than compute units (M = 128 and M = 512 at N = 28672
have 224 tiles for 256 CUs) the consumer deals equal runs of (tile, shard)
units to the workgroups; a tile whose shards fall to several workgroups is
summed by the last of them, in a fixed contributor order. The sum over shards
is the AG+GEMM core identity ("Eliminating Multi-GPU Performance Taxes"
analysis page); any grouping of it is an equally correct result, so the bar
is the oracle's: bit for bit on exact inputs, within 1e-3*sqrt(K) otherwise,
and identical C from the fused, BSP and pull paths of one context.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _ctx(W, M, K, N, c_dtype="f32"):
    from shard_decomposed_gemm_amd import Context
    return Context(W, M, K, N, c_dtype=c_dtype)


def _paths(ctx, dsh, B, c_dtype, schedule):
    import torch
    out = {}
    sp, sc = ctx.streams()
    C = gu.empty_c(ctx.M, ctx.N, c_dtype)
    ctx.produce(dsh, schedule=schedule, stream=sp)
    ctx.run_fused(B, C, stream=sc)
    out["fused"] = C
    C = gu.empty_c(ctx.M, ctx.N, c_dtype)
    ctx.run_bsp(dsh, B, C, schedule=schedule, host_sync=True)
    out["bsp"] = C
    C = gu.empty_c(ctx.M, ctx.N, c_dtype)
    ctx.run_pull(dsh, B, C)
    out["pull"] = C
    torch.cuda.synchronize()
    ctx.check()
    return out


@pytest.mark.parametrize("M,N,K,split", [(128, 28672, 8192, False), (512, 28672, 8192, False),
                                         (4096, 28672, 8192, False), (128, 4096, 8192, True),
                                         (512, 2048, 8192, True), (128, 4096, 2048, False), (8, 256, 512, False)])
def test_plan(M, N, K, split):
    """The automatic choice at W = 8: the workloads' 224 and 1792 tiles keep whole tiles
    (224 tiles on 256 CUs: the hand-off of the partials costs more than the shorter run);
    at K = 8192, 32 tiles (M = 128, N = 4096) and 16 tiles (M = 512, N = 2048) split, over
    one workgroup per CU or one per (tile, shard) unit if there are fewer; at K = 2048 and
    on the tiny workload the split would save too little of K and whole tiles stay."""
    import torch
    ctx = _ctx(8, M, K, N, "f16")
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    assert ctx.consumer[0] == "mfma"
    assert ctx.split is split
    info = ctx.consumer_info()
    tiles = -(-M // info["block_m"]) * -(-N // info["block_n"])
    split_cus = n_cu if info["tile_config"] == 1 else n_cu - n_cu // 8
    assert ctx.grid == (min(split_cus, tiles * 8) if split else min(n_cu, tiles))
    ctx.close()


@pytest.mark.parametrize("mode", ["0", "1"])
@pytest.mark.parametrize("tile_config", [0, 1, 2])
@pytest.mark.parametrize("W,M,K,N", [
    (8, 300, 2048, 1032),   # 10 tiles x 8 shards: many contributors per tile
    (4, 520, 1024, 264),    # 6 tiles x 4 shards, ragged rows and columns
    (16, 130, 1024, 4104),  # 16 shards of one k-step each
    (3, 257, 768, 776),     # W = 3: runs cut at uneven shard counts
])
def test_split_exact_bitwise(W, M, K, N, tile_config, mode, monkeypatch):
    """Exact inputs (every product and partial sum exact in fp32): split and whole-tile
    results must both equal the oracle bit for bit (fp32 C) or its round-to-nearest-even
    (fp16 C), on every path, with the producer releasing tiles out of order while the
    fused consumer runs."""
    monkeypatch.setenv("AGEMM_TILE_CONFIG", str(tile_config))
    monkeypatch.setenv("AGEMM_SPLIT", mode)
    a = gu.coarse_bits(0xF000 + M, M, K)
    b = gu.coarse_bits(0xF100 + N, K, N)
    sh = synth.shards(a, W)
    ref = oracle.sharded_gemm(sh, b)
    dsh = [gu.to_dev(s) for s in sh]
    B = gu.to_dev(b)
    for c_dtype in ("f32", "f16"):
        ctx = _ctx(W, M, K, N, c_dtype)
        assert ctx.split is (mode == "1")
        sched = synth.schedule(0xF200 + tile_config, ctx.t, 8_000)
        outs = _paths(ctx, dsh, B, c_dtype, sched)
        for path, C in outs.items():
            if c_dtype == "f32":
                assert np.array_equal(C.cpu().numpy().astype(np.float64), ref), (path, tile_config, mode)
            else:
                assert np.array_equal(C.cpu().numpy().view(np.uint16), ref.astype(np.float16).view(np.uint16)), \
                    (path, tile_config, mode)
        ctx.close()


@pytest.mark.parametrize("c_dtype", ["f16", "f32"])
@pytest.mark.parametrize("W,M,K,N", [(8, 200, 4096, 3080), (8, 129, 2048, 6152), (2, 700, 1024, 1000)])
def test_split_random_against_oracle(W, M, K, N, c_dtype, monkeypatch):
    """Random inputs: the split result is within the oracle's tolerance, the three paths
    agree bit for bit, and the whole-tile result of a second context is within the
    tolerance too (the two group the shard sum differently)."""
    import torch
    a, sh, b, dsh, B = gu.random_problem(W, M, K, N, seed=0x51 + M)
    ref = oracle.sharded_gemm(sh, b)
    tol = oracle.tolerance(K)
    monkeypatch.setenv("AGEMM_SPLIT", "1")
    ctx = _ctx(W, M, K, N, c_dtype)
    assert ctx.split
    outs = _paths(ctx, dsh, B, c_dtype, synth.schedule(0x5A00 + M, ctx.t, 5_000))
    iv = (lambda C: C.view(torch.int16)) if c_dtype == "f16" else (lambda C: C.view(torch.int32))
    assert torch.equal(iv(outs["fused"]), iv(outs["bsp"]))
    assert torch.equal(iv(outs["fused"]), iv(outs["pull"]))
    got = gu.c_to_f64(outs["fused"])
    assert np.isfinite(got).all()
    assert np.abs(got - ref).max() <= tol
    ctx.close()
    monkeypatch.setenv("AGEMM_SPLIT", "0")
    ctx0 = _ctx(W, M, K, N, c_dtype)
    assert not ctx0.split
    C0 = gu.empty_c(M, N, c_dtype)
    ctx0.run_pull(dsh, B, C0)
    torch.cuda.synchronize()
    assert np.abs(gu.c_to_f64(C0) - ref).max() <= tol
    ctx0.close()


def test_split_back_to_back_calls_reuse_counters(monkeypatch):
    """Forty consumer calls in a row on one context, alternating two data sets and the
    three paths: the hand-off counters are cleared by each tile's last contributor, so
    every call must reproduce its data set's first result bit for bit."""
    import torch
    monkeypatch.setenv("AGEMM_SPLIT", "1")
    W, M, K, N = 8, 384, 2048, 2056
    probs = [gu.random_problem(W, M, K, N, seed=s) for s in (0x61, 0x62)]
    ctx = _ctx(W, M, K, N, "f16")
    assert ctx.split
    refs = []
    for p in probs:
        C = gu.empty_c(M, N, "f16")
        ctx.run_pull(p[3], p[4], C)
        refs.append(C)
    torch.cuda.synchronize()
    assert np.abs(gu.c_to_f64(refs[0]) - oracle.sharded_gemm(probs[0][1], probs[0][2])).max() <= oracle.tolerance(K)
    sp, sc = ctx.streams()
    bad = []
    for i in range(40):
        p = probs[i % 2]
        C = gu.empty_c(M, N, "f16")
        kind = i % 3
        if kind == 0:
            ctx.produce(p[3], stream=sp)
            ctx.run_fused(p[4], C, stream=sc)
        elif kind == 1:
            ctx.run_bsp(p[3], p[4], C, host_sync=False, stream=sc)
        else:
            ctx.run_pull(p[3], p[4], C, stream=sc)
        torch.cuda.synchronize()
        if not torch.equal(C.view(torch.int16), refs[i % 2].view(torch.int16)):
            bad.append(i)
    ctx.check()
    assert not bad, bad
    ctx.close()


def test_arrival_order_on_a_split_context_runs_whole_tiles(monkeypatch):
    """A context that runs the split (10 tiles) asked for arrival order: those fused
    calls run on whole tiles in arrival order, bit-exact against the oracle on exact
    inputs, with tiles released out of order into a poisoned inbox; shard-order calls
    on the same context still split."""
    import torch
    monkeypatch.setenv("AGEMM_SPLIT", "1")
    W, M, K, N = 8, 300, 2048, 1032
    a = gu.coarse_bits(0xF700 + M, M, K)
    b = gu.coarse_bits(0xF800 + N, K, N)
    sh = synth.shards(a, W)
    ref = oracle.sharded_gemm(sh, b)
    dsh = [gu.to_dev(s) for s in sh]
    B = gu.to_dev(b)
    ctx = _ctx(W, M, K, N, "f32")
    assert ctx.split
    nan = [torch.full((M, K // W), float("nan"), dtype=torch.float16, device=gu.dev()) for _ in range(W)]
    ctx.produce(nan)
    ctx.produce(nan)
    torch.cuda.synchronize()
    sp, sc = ctx.streams()
    for order in ("arrival", "shard", "arrival"):
        ctx.set_order(order)
        sched = synth.schedule(0xF900 + len(order), ctx.t, 10_000)
        C = gu.empty_c(M, N, "f32")
        ctx.produce(dsh, schedule=sched, stream=sp)
        ctx.run_fused(B, C, stream=sc)
        torch.cuda.synchronize()
        ctx.check()
        assert np.array_equal(C.cpu().numpy().astype(np.float64), ref), order
    ctx.close()


def test_inbox_guard_counts_with_changing_grids():
    """Fused launches of one context count different numbers of units into the inbox
    guard: the split (one workgroup per CU) in shard order, whole tiles (32
    workgroups) in arrival order. Alternating the two over pipelined epochs on the
    context's stream pair, with no synchronisation between epochs, every producer must
    find exactly the counts its inbox's earlier launches raise (a total too high
    would hold it until the spin timeout), and every epoch's C must equal the oracle
    bit for bit (exact inputs: any summation order gives the same C)."""
    import torch
    W, M, K, N = 8, 128, 8192, 4096
    sets = []
    for k in range(3):
        a = gu.coarse_bits(0xFA00 + k, M, K)
        b = gu.coarse_bits(0xFB00 + k, K, N)
        sh = synth.shards(a, W)
        sets.append((oracle.sharded_gemm(sh, b), [gu.to_dev(s) for s in sh], gu.to_dev(b)))
    ctx = _ctx(W, M, K, N, "f32")
    assert ctx.split and ctx.consumer_info()["tile_config"] == 1
    sp, sc = ctx.streams()
    outs = []
    for e in range(6):
        ctx.set_order("arrival" if e % 2 else "shard")
        ref, dsh, B = sets[e % 3]
        C = gu.empty_c(M, N, "f32")
        ctx.produce(dsh, schedule=synth.schedule(0xFC00 + e, ctx.t, 5_000), stream=sp)
        ctx.run_fused(B, C, stream=sc)
        outs.append(C)
    torch.cuda.synchronize()
    ctx.check()
    for e, C in enumerate(outs):
        assert np.array_equal(C.cpu().numpy().astype(np.float64), sets[e % 3][0]), e
    ctx.close()
