"""GPU parity: the HIP path (through the C-ABI) against the CPU oracle.

Bar: max |C_gpu - C_oracle| <= 1e-3 * sqrt(K) for fp16 inputs uniform in
[-1, 1] with fp32 accumulation (fp16 or fp32 C); bit-exact on inputs whose
products and partial sums are exact in fp32 (every summation order then gives
the same fp32 value).
"""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _ctx(W, M, K, N, c_dtype, **kw):
    from shard_decomposed_gemm_amd import Context
    return Context(W, M, K, N, c_dtype=c_dtype, **kw)


def _run(ctx, path, shards, B, C, schedule=None):
    import torch
    if path == "fused":
        sp, sc = ctx.streams()
        ctx.produce(shards, schedule=schedule, stream=sp)
        ctx.run_fused(B, C, stream=sc)
    elif path == "fused_preset":
        ctx.produce(shards, schedule=schedule)
        torch.cuda.synchronize()
        ctx.run_fused(B, C)
    elif path == "bsp":
        ctx.run_bsp(shards, B, C, schedule=schedule, host_sync=True)
    elif path == "bsp_nosync":
        ctx.run_bsp(shards, B, C, schedule=schedule, host_sync=False)
    elif path == "pull":
        ctx.run_pull(shards, B, C)
    else:
        raise ValueError(path)
    torch.cuda.synchronize()
    ctx.check()


def test_tiny_config_flags_preset():
    """W=8, M=8, K=512, N=256, fp32 C, every flag raised before the consumer starts."""
    W, M, K, N = 8, 8, 512, 256
    a, sh, b, dsh, B = gu.random_problem(W, M, K, N, seed=1)
    ref = oracle.sharded_gemm(sh, b)
    ctx = _ctx(W, M, K, N, "f32")
    C = gu.empty_c(M, N, "f32")
    _run(ctx, "fused_preset", dsh, B, C)
    err = np.abs(gu.c_to_f64(C) - ref).max()
    assert err <= oracle.tolerance(K), err


@pytest.mark.parametrize("path", ["fused", "fused_preset", "bsp", "pull"])
@pytest.mark.parametrize("c_dtype", ["f32", "f16"])
def test_tiny_config_against_stored_golden(path, c_dtype):
    """The tiny workload against the exact C stored in tests/golden/ (written from the
    oracle by tests/golden/make_golden.py), not against a live oracle call."""
    from tests import golden_io
    W, M, K, N = 8, 8, 512, 256
    _, _, _, dsh, B = gu.random_problem(W, M, K, N, seed=1)
    ctx = _ctx(W, M, K, N, c_dtype)
    C = gu.empty_c(M, N, c_dtype)
    _run(ctx, path, dsh, B, C)
    err = np.abs(gu.c_to_f64(C) - golden_io.tiny_c()).max()
    assert err <= oracle.tolerance(K), err


SHAPES = [
    # W, M, K, N                      kernel exercised (default choice)
    (8, 8, 512, 256),                 # 128x128 MFMA tiles, stream-K split, tiny workload
    (8, 1, 2048, 1000),               # small-M, ragged column block
    (4, 3, 1024, 4104),               # 128x128 MFMA tiles, M not a power of two
    (2, 7, 256, 72),                  # 128x128 MFMA tile, W = 2, one ragged tile
    (8, 130, 2048, 520),              # 128x128 MFMA tiles, ragged rows and columns
    (1, 40, 512, 136),                # W = 1 (no decomposition)
    (8, 300, 2048, 1000),             # 256x256 MFMA tiles, ragged rows and columns
    (16, 257, 1024, 264),             # 16 shards of 64 columns, one row over a tile
]


@pytest.mark.parametrize("W,M,K,N", SHAPES)
@pytest.mark.parametrize("path", ["fused", "bsp", "pull"])
@pytest.mark.parametrize("c_dtype", ["f16", "f32"])
def test_parity_random(W, M, K, N, path, c_dtype):
    a, sh, b, dsh, B = gu.random_problem(W, M, K, N, seed=W * 7 + M)
    ref = oracle.sharded_gemm(sh, b)
    ctx = _ctx(W, M, K, N, c_dtype)
    C = gu.empty_c(M, N, c_dtype)
    _run(ctx, path, dsh, B, C)
    got = gu.c_to_f64(C)
    assert np.isfinite(got).all()
    err = np.abs(got - ref).max()
    assert err <= oracle.tolerance(K), (err, oracle.tolerance(K))


@pytest.mark.parametrize("W,M,K,N", SHAPES)
@pytest.mark.parametrize("path", ["fused", "bsp", "pull"])
def test_parity_exact_inputs(W, M, K, N, path):
    """Inputs on a 1/16 grid: fp32 accumulation is exact, so C must equal the oracle bit for bit
    (fp32 C), and fp16 C must be its round-to-nearest-even."""
    a = gu.coarse_bits(0xC000 + M, M, K)
    b = gu.coarse_bits(0xC100 + N, K, N)
    sh = synth.shards(a, W)
    ref = oracle.sharded_gemm(sh, b)
    assert np.array_equal(ref.astype(np.float32).astype(np.float64), ref)  # exact in fp32
    dsh = [gu.to_dev(s) for s in sh]
    B = gu.to_dev(b)
    for c_dtype in ("f32", "f16"):
        ctx = _ctx(W, M, K, N, c_dtype)
        C = gu.empty_c(M, N, c_dtype)
        _run(ctx, path, dsh, B, C)
        if c_dtype == "f32":
            assert np.array_equal(C.cpu().numpy().astype(np.float64), ref)
        else:
            assert np.array_equal(C.cpu().numpy().view(np.uint16), ref.astype(np.float16).view(np.uint16))


# The small-M streaming kernel takes M up to 8 when asked (AGEMM_SMALL_M_MAX); by
# default it runs at M = 1 only.
SMALL_M_SHAPES = [
    (8, 8, 512, 256),                 # tiny workload
    (8, 2, 2048, 1000),               # ragged column block
    (4, 3, 1024, 4104),               # M not a power of two
    (2, 7, 256, 72),                  # W = 2
    (16, 5, 2048, 264),               # 16 shards
]


@pytest.mark.parametrize("W,M,K,N", SMALL_M_SHAPES)
@pytest.mark.parametrize("path", ["fused", "bsp", "pull"])
def test_small_m_kernel_up_to_m8(W, M, K, N, path, monkeypatch):
    """The small-M kernel at 1 < M <= 8: uniform inputs within the tolerance (fp16 and
    fp32 C), and exact inputs bit for bit."""
    gu.pick_consumer(monkeypatch, "small_m")
    a, sh, b, dsh, B = gu.random_problem(W, M, K, N, seed=W * 11 + M)
    ref = oracle.sharded_gemm(sh, b)
    for c_dtype in ("f16", "f32"):
        ctx = _ctx(W, M, K, N, c_dtype)
        gu.assert_consumer(ctx, "small_m")
        C = gu.empty_c(M, N, c_dtype)
        _run(ctx, path, dsh, B, C)
        assert np.abs(gu.c_to_f64(C) - ref).max() <= oracle.tolerance(K), c_dtype
    a = gu.coarse_bits(0xC200 + M, M, K)
    b = gu.coarse_bits(0xC300 + N, K, N)
    sh = synth.shards(a, W)
    ref = oracle.sharded_gemm(sh, b)
    ctx = _ctx(W, M, K, N, "f32")
    C = gu.empty_c(M, N, "f32")
    _run(ctx, path, [gu.to_dev(s) for s in sh], gu.to_dev(b), C)
    assert np.array_equal(C.cpu().numpy().astype(np.float64), ref)


def test_default_consumer_by_m(monkeypatch):
    """The small-M kernel is the default at M = 1 only; AGEMM_SMALL_M_MAX moves the cutoff
    (0: never, up to 8)."""
    W, K, N = 8, 1024, 1024
    for M, kind in ((1, "small_m"), (2, "mfma"), (8, "mfma"), (9, "mfma")):
        ctx = _ctx(W, M, K, N, "f16")
        assert ctx.consumer_info()["kind"] == kind, (M, ctx.consumer_info())
        ctx.close()
    monkeypatch.setenv("AGEMM_SMALL_M_MAX", "0")
    ctx = _ctx(W, 1, K, N, "f16")
    assert ctx.consumer_info()["kind"] == "mfma"
    ctx.close()
    monkeypatch.setenv("AGEMM_SMALL_M_MAX", "8")
    for M, kind in ((8, "small_m"), (9, "mfma")):
        ctx = _ctx(W, M, K, N, "f16")
        assert ctx.consumer_info()["kind"] == kind, (M, ctx.consumer_info())
        ctx.close()


@pytest.mark.parametrize("M", [1, 8, 200, 512])
def test_structural_closed_forms(M):
    """One-hot rows select B rows; A living in one shard sees only that shard's B rows;
    B of ones gives every column the row sums of A; A = 0 gives C = 0."""
    import torch
    W, K, N = 8, 2048, 776
    KS = K // W
    b = synth.matrix_f16(0xB0B0, K, N)
    B = gu.to_dev(b)
    one = np.uint16(0x3C00)
    picks = [(m * 131 + (m % 3) * KS - 1) % K for m in range(M)]
    picks[0] = KS - 1          # last column of shard 0
    if M > 1:
        picks[1] = KS          # first column of shard 1
    a = np.zeros((M, K), dtype=np.uint16)
    for m, k in enumerate(picks):
        a[m, k] = one
    ctx = _ctx(W, M, K, N, "f32")
    C = gu.empty_c(M, N, "f32")
    _run(ctx, "fused", [gu.to_dev(s) for s in synth.shards(a, W)], B, C)
    got = C.cpu().numpy()
    bf = b.view(np.float16).astype(np.float32)
    for m, k in enumerate(picks):
        assert np.array_equal(got[m], bf[k]), m
    # A supported on shard 3 only
    a2 = np.zeros((M, K), dtype=np.uint16)
    a2[:, 3 * KS:4 * KS] = gu.coarse_bits(0xD0D0, M, KS)
    sh2 = synth.shards(a2, W)
    C2 = gu.empty_c(M, N, "f32")
    _run(ctx, "fused", [gu.to_dev(s) for s in sh2], B, C2)
    ref = oracle.shard_partial(sh2, b, 3)
    assert np.abs(C2.cpu().numpy().astype(np.float64) - ref).max() <= oracle.tolerance(K)
    # B = 1 -> C[m, n] = sum_k A[m, k] for every n (exact: A on a 1/16 grid, |sum| <= K)
    a4 = gu.coarse_bits(0xD1D1, M, K)
    ones = np.full((K, N), one, dtype=np.uint16)
    C4 = gu.empty_c(M, N, "f32")
    _run(ctx, "fused", [gu.to_dev(s) for s in synth.shards(a4, W)], gu.to_dev(ones), C4)
    rows = a4.view(np.float16).astype(np.float64).sum(axis=1)
    assert np.array_equal(C4.cpu().numpy().astype(np.float64), np.repeat(rows[:, None], N, axis=1))
    # A = 0 -> C = 0
    C3 = gu.empty_c(M, N, "f32")
    _run(ctx, "fused", [torch.zeros((M, KS), dtype=torch.float16, device=gu.dev()) for _ in range(W)], B, C3)
    assert not C3.cpu().numpy().any()


@pytest.mark.parametrize("tile_config", [0, 1, 2])
@pytest.mark.parametrize("W,M,K,N", [(8, 300, 2048, 1032), (4, 520, 1024, 264)])
def test_every_tile_config(tile_config, W, M, K, N, monkeypatch):
    """Each MFMA tile configuration (chosen at create time through AGEMM_TILE_CONFIG),
    gated with the producer running concurrently, ungated (pull) and BSP, on ragged
    shapes: exact inputs, so fused, BSP and pull must agree bit for bit with the oracle."""
    monkeypatch.setenv("AGEMM_TILE_CONFIG", str(tile_config))
    a = gu.coarse_bits(0xE000 + M, M, K)
    b = gu.coarse_bits(0xE100 + N, K, N)
    sh = synth.shards(a, W)
    ref = oracle.sharded_gemm(sh, b)
    dsh = [gu.to_dev(s) for s in sh]
    B = gu.to_dev(b)
    ctx = _ctx(W, M, K, N, "f32")
    order, offs = synth.schedule(0xE200 + tile_config, ctx.t, 10_000)
    for path in ("fused", "pull", "bsp"):
        C = gu.empty_c(M, N, "f32")
        _run(ctx, path, dsh, B, C, schedule=(order, offs) if path != "pull" else None)
        assert np.array_equal(C.cpu().numpy().astype(np.float64), ref), (tile_config, path)


def test_kernel_timing_events():
    """agemm_timing_begin/end: one duration per consumer launch (capped), in launch
    order, positive; end without begin is a state error."""
    import torch
    from shard_decomposed_gemm_amd import AgemmError
    from shard_decomposed_gemm_amd.agemm import ESTATE
    W, M, K, N = 8, 130, 2048, 520
    a, sh, b, dsh, B = gu.random_problem(W, M, K, N, seed=91)
    ctx = _ctx(W, M, K, N, "f32")
    C = gu.empty_c(M, N, "f32")
    ctx.timing_begin(2)
    for _ in range(3):
        ctx.produce(dsh)
        ctx.run_fused(B, C)
    ctx.run_pull(dsh, B, C)
    torch.cuda.synchronize()
    us = ctx.timing_end()
    assert len(us) == 2 and all(0.0 < u < 1e6 for u in us), us
    with pytest.raises(AgemmError) as ei:
        ctx.timing_end()
    assert ei.value.status == ESTATE
    ctx.check()
    assert np.abs(gu.c_to_f64(C) - oracle.sharded_gemm(sh, b)).max() <= oracle.tolerance(K)
