"""Element-wise oracle parity for the consumer launches the full-size workloads run.

The full-size workloads run launch shapes that small parity shapes do not
reach: more output tiles than workgroups (a persistent workgroup runs several
tiles and its load cursor crosses from one tile into the next), the XCD-aware
tile order with its groups of 8 row blocks (ragged last group), and the
nontemporal-B loads used when C has one row block. These cases reach the
same launch shapes at a small K, where the oracle checks every entry of C.

Each case first asserts, through agemm_consumer_info, that the context
launches the intended kernel (tile configuration, tiles per workgroup, split,
B load policy). Inputs on a 1/16 grid make every fp32 partial sum exact, so
fp32 C must equal the oracle bit for bit and fp16 C must be its
round-to-nearest-even, whatever the path and order; random uniform[-1, 1]
inputs are held to max|err| <= 1e-3 * sqrt(K) (the analysis page's AG+GEMM
core identity; every k-tile of every output tile over all shards, as its
correctness check #3 requires of the tiled loop).
"""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

NUM_CUS = 256  # MI355X

CASES = {
    # name: (W, M, K, N, expected consumer launch)
    # 256x256 tiles: 9 x 32 = 288 tiles on 256 workgroups, XCD order on, two row-block
    # groups (8 + a ragged 1), ragged last rows and columns
    "t256_xcd_groups": (8, 2100, 512, 8184,
                        dict(kind="mfma", tile_config=0, tiles=288, grid=256, split=0, tiles_per_wg=2,
                             b_nontemporal=0, a_panels=1)),
    # 256x256 tiles: 4 x 66 = 264 tiles, K = 1024 (two k-tiles per shard)
    "t256_k1024": (8, 1000, 1024, 16888,
                   dict(kind="mfma", tile_config=0, tiles=264, grid=256, split=0, tiles_per_wg=2,
                        b_nontemporal=0, a_panels=1)),
    # 256x128 tiles, one row block (M just over 128, ragged rows): nontemporal B,
    # 160 workgroups of one tile each
    "t256x128_nontemporal_b": (8, 130, 512, 20480,
                               dict(kind="mfma", tile_config=2, tiles=160, grid=160, split=0, tiles_per_wg=1,
                                    b_nontemporal=1, a_panels=1)),
    # 256x128 tiles, one row block, 300 tiles on 256 workgroups: the cursor crosses
    # tiles, ragged last columns
    "t256x128_persistent": (8, 256, 512, 38392,
                            dict(kind="mfma", tile_config=2, tiles=300, grid=256, split=0, tiles_per_wg=2,
                                 b_nontemporal=1, a_panels=1)),
    # 128x128 tiles, one row block: nontemporal B, 160 workgroups of one tile each
    "t128_nontemporal_b": (8, 96, 1024, 20472,
                           dict(kind="mfma", tile_config=1, tiles=160, grid=160, split=0, tiles_per_wg=1,
                                b_nontemporal=1, a_panels=1)),
    # 128x128 tiles, one row block, 288 tiles on 256 workgroups: nontemporal B with the
    # cursor crossing tiles
    "t128_nontemporal_b_persistent": (8, 100, 512, 36864,
                                      dict(kind="mfma", tile_config=1, tiles=288, grid=256, split=0,
                                           tiles_per_wg=2, b_nontemporal=1, a_panels=1)),
}

_cache = {}


def _exact_problem(name):
    """Inputs on a 1/16 grid and the oracle's C (computed once per case)."""
    if name not in _cache:
        W, M, K, N, _ = CASES[name]
        a = gu.coarse_bits(0xD000 + M, M, K)
        b = gu.coarse_bits(0xD100 + N, K, N)
        sh = synth.shards(a, W)
        ref = oracle.sharded_gemm(sh, b)
        assert np.array_equal(ref.astype(np.float32).astype(np.float64), ref)  # exact in fp32
        _cache[name] = (sh, b, ref)
    return _cache[name]


def _check_launch(ctx, expect):
    from shard_decomposed_gemm_amd import agemm
    if agemm.device_info()["cus"] != NUM_CUS:
        pytest.skip("launch shapes are stated for a 256-CU MI355X")
    info = ctx.consumer_info()
    for k, v in expect.items():
        assert info[k] == v, (k, info)


def _poison(ctx, W, M, K):
    """Fill both inboxes with fp16 NaN (two epochs): a read before a flag shows up as NaN."""
    import torch
    nan = [torch.full((M, K // W), float("nan"), dtype=torch.float16, device=gu.dev()) for _ in range(W)]
    ctx.produce(nan)
    ctx.produce(nan)
    torch.cuda.synchronize()


def _run(ctx, path, dsh, B, C, sched):
    import torch
    if path in ("fused", "fused_arrival"):
        sp, sc = ctx.streams()
        ctx.produce(dsh, schedule=sched, stream=sp)
        ctx.run_fused(B, C, stream=sc)
    elif path == "bsp":
        ctx.run_bsp(dsh, B, C, schedule=sched, host_sync=True)
    elif path == "pull":
        ctx.run_pull(dsh, B, C)
    torch.cuda.synchronize()
    ctx.check()


@pytest.mark.parametrize("path", ["fused", "fused_arrival", "bsp", "pull"])
@pytest.mark.parametrize("name", list(CASES))
def test_every_entry_exact(name, path):
    """Every entry of C, bit for bit, for fp32 and fp16 C. The fused paths release the
    flag tiles in a seeded random order with delays into inboxes full of NaN."""
    from shard_decomposed_gemm_amd import Context
    W, M, K, N, expect = CASES[name]
    sh, b, ref = _exact_problem(name)
    dsh = [gu.to_dev(s) for s in sh]
    B = gu.to_dev(b)
    print(f"[tiled-parity] {name} path={path} W={W} M={M} K={K} N={N}", flush=True)
    for c_dtype in ("f32", "f16"):
        ctx = Context(W, M, K, N, c_dtype=c_dtype)
        if path == "fused_arrival":
            ctx.set_order("arrival")
            # arrival order keeps the default B policy
            _check_launch(ctx, dict(expect, b_nontemporal=0))
        else:
            _check_launch(ctx, expect)
        sched = None
        if path.startswith("fused"):
            _poison(ctx, W, M, K)
            sched = synth.schedule(0x5400 + M, ctx.t, 5_000)
        C = gu.empty_c(M, N, c_dtype)
        _run(ctx, path, dsh, B, C, sched)
        if c_dtype == "f32":
            got = C.cpu().numpy().astype(np.float64)
            bad = np.argwhere(got != ref)
            assert bad.size == 0, (bad[:5], got[tuple(bad[0])], ref[tuple(bad[0])])
        else:
            want = ref.astype(np.float16).view(np.uint16)
            got = C.cpu().numpy().view(np.uint16)
            bad = np.argwhere(got != want)
            assert bad.size == 0, bad[:5]
        ctx.close()


@pytest.mark.parametrize("name", list(CASES))
def test_random_inputs_within_tolerance(name):
    """uniform[-1, 1] inputs, fused path (out-of-order release, poisoned inboxes), fp16 C."""
    from shard_decomposed_gemm_amd import Context
    W, M, K, N, expect = CASES[name]
    a, sh, b, dsh, B = gu.random_problem(W, M, K, N, seed=0x31 + M)
    ref = oracle.sharded_gemm(sh, b)
    print(f"[tiled-parity] random {name}", flush=True)
    ctx = Context(W, M, K, N, c_dtype="f16")
    _check_launch(ctx, expect)
    _poison(ctx, W, M, K)
    C = gu.empty_c(M, N, "f16")
    _run(ctx, "fused", dsh, B, C, synth.schedule(0x5500 + M, ctx.t, 5_000))
    got = gu.c_to_f64(C)
    assert np.isfinite(got).all()
    err = np.abs(got - ref).max()
    assert err <= oracle.tolerance(K), err
    ctx.close()
