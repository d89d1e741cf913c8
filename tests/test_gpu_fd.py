"""GPU parity of the flag-gated Flash-Decode combine against the CPU oracle.

"Eliminating Multi-GPU Performance Taxes" analysis page: Flash Decode global
reduction (online-softmax combine of the W ranks' partials) and correctness
check #5 (any combine order). Bar: |O_gpu - O_oracle| <= oracle.fd.tolerance
(binary32 arithmetic, W <= 16 partials in [-1, 1]); bit for bit on inputs
whose combine is exact in binary32 (equal statistics, coarse outputs, W a
power of two).
"""
import numpy as np
import pytest

import synth
from oracle import fd as fdo
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _dev_parts(o, lse):
    import torch
    return ([torch.from_numpy(np.ascontiguousarray(x)).to(gu.dev()) for x in o],
            [torch.from_numpy(np.ascontiguousarray(x)).to(gu.dev()) for x in lse])


def _out(H, D, dtype):
    import torch
    dt = torch.float16 if dtype == "f16" else torch.float32
    return torch.full((H, D), float("nan"), dtype=dt, device=gu.dev())


def _ctx(W, H, D, HT, dtype):
    from shard_decomposed_gemm_amd import FdCombine
    return FdCombine(W, H, D, heads_per_tile=HT, out_dtype=dtype)


def _fused(ctx, o, lse, O, schedule=None):
    import torch
    sp, sc = ctx.streams()
    ctx.produce(o, lse, schedule=schedule, stream=sp)
    ctx.run_fused(O, stream=sc)
    torch.cuda.synchronize()
    ctx.check()


SHAPES = [
    # W, H, D, HT
    (8, 96, 128, 16),   # the pages' Flash-Decode shape: 96 heads, d = 128, 8 ranks
    (8, 96, 128, 12),   # 64 tiles
    (1, 32, 64, 8),     # one rank: the combine is the identity
    (16, 64, 256, 16),  # 16 ranks, d = 256
    (3, 20, 128, 4),    # odd rank count, heads not a multiple of 4 waves
    (2, 1024, 64, 32),  # the largest head tile (32 heads per flag), 1024 heads, T = 64
]


@pytest.mark.parametrize("W,H,D,HT", SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("path", ["fused", "bsp"])
def test_fd_parity_random(W, H, D, HT, dtype, path):
    o, lse = synth.fd_partials(0x7200 + W * 100 + H, W, H, D)
    ref = fdo.combine(o, lse)
    do, dl = _dev_parts(o, lse)
    ctx = _ctx(W, H, D, HT, dtype)
    order, offs = synth.schedule(0x7300 + H, ctx.t, 20_000)
    O = _out(H, D, dtype)
    if path == "fused":
        _fused(ctx, do, dl, O, (order, offs))
    else:
        import torch
        ctx.run_bsp(do, dl, O, schedule=(order, offs), host_sync=True)
        torch.cuda.synchronize()
        ctx.check()
    got = O.float().cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    assert np.abs(got - ref).max() <= fdo.tolerance(dtype)


@pytest.mark.parametrize("path", ["fused", "bsp"])
def test_fd_exact_inputs_bitwise(path):
    """Equal statistics across ranks and outputs on a 1/16 grid: every weight is 1 and
    every sum exact, so any combine order gives the oracle's mean bit for bit."""
    import torch
    W, H, D, HT = 8, 96, 128, 16
    o, _ = synth.fd_partials(0x7400, W, H, D)
    o = [np.rint(x * 16.0) / 16.0 for x in o]
    o = [x.astype(np.float32) for x in o]
    lse = [np.full(H, 11.5, dtype=np.float32) + np.arange(H, dtype=np.float32) * 0.25 for _ in range(W)]
    ref = fdo.combine(o, lse)
    do, dl = _dev_parts(o, lse)
    ctx = _ctx(W, H, D, HT, "f32")
    O = _out(H, D, "f32")
    order, offs = synth.schedule(0x7401, ctx.t, 10_000)
    if path == "fused":
        _fused(ctx, do, dl, O, (order, offs))
    else:
        ctx.run_bsp(do, dl, O, schedule=(order, offs))
        torch.cuda.synchronize()
    assert np.array_equal(O.cpu().numpy().astype(np.float64), ref)


@pytest.mark.parametrize("path", ["fused", "bsp"])
def test_fd_against_stored_golden(path):
    """W=4, H=16, d=64 against the binary64 O stored in tests/golden/ (written from
    the oracle by tests/golden/make_golden.py)."""
    import torch
    from tests import golden_io
    W, H, D, HT = 4, 16, 64, 8
    o, lse = synth.fd_partials(0x7A00, W, H, D)
    do, dl = _dev_parts(o, lse)
    ctx = _ctx(W, H, D, HT, "f32")
    O = _out(H, D, "f32")
    if path == "fused":
        _fused(ctx, do, dl, O)
    else:
        ctx.run_bsp(do, dl, O)
        torch.cuda.synchronize()
        ctx.check()
    got = O.cpu().numpy().astype(np.float64)
    assert np.abs(got - golden_io.fd()).max() <= fdo.tolerance("f32")


def test_fd_poisoned_inbox_is_never_read_early():
    """Both inboxes hold NaN partials from two earlier epochs; the real epoch releases
    its tiles out of order, up to 40 us apart, while the combine already runs."""
    import torch
    W, H, D, HT = 8, 96, 128, 16
    o, lse = synth.fd_partials(0x7500, W, H, D)
    ref = fdo.combine(o, lse)
    do, dl = _dev_parts(o, lse)
    ctx = _ctx(W, H, D, HT, "f32")
    nan_o = [torch.full((H, D), float("nan"), device=gu.dev()) for _ in range(W)]
    nan_l = [torch.full((H,), float("nan"), device=gu.dev()) for _ in range(W)]
    ctx.produce(nan_o, nan_l)
    ctx.produce(nan_o, nan_l)
    torch.cuda.synchronize()
    order, offs = synth.schedule(0x7501, ctx.t, 40_000)
    O = _out(H, D, "f32")
    _fused(ctx, do, dl, O, (order, offs))
    got = O.cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    assert np.abs(got - ref).max() <= fdo.tolerance("f32")


def test_fd_alternating_epochs():
    """Three data sets cycle over six epochs on two streams: each epoch's output matches
    its own partials (an inbox is not overwritten while a combine still reads it)."""
    import torch
    W, H, D, HT = 8, 96, 128, 16
    sets = [synth.fd_partials(0x7600 + 16 * k, W, H, D) for k in range(3)]
    refs = [fdo.combine(o, l) for o, l in sets]
    devs = [_dev_parts(o, l) for o, l in sets]
    ctx = _ctx(W, H, D, HT, "f32")
    sp, sc = ctx.streams()
    outs = []
    for e in range(6):
        k = e % 3
        order, offs = synth.schedule(0x7700 + e, ctx.t, 5_000 if e % 2 else 0)
        O = _out(H, D, "f32")
        ctx.produce(*devs[k], schedule=(order, offs), stream=sp)
        ctx.run_fused(O, stream=sc)
        outs.append(O)
    torch.cuda.synchronize()
    ctx.check()
    for e, O in enumerate(outs):
        assert np.abs(O.cpu().numpy().astype(np.float64) - refs[e % 3]).max() <= fdo.tolerance("f32"), e


def test_fd_epochs_across_the_counter_wrap(monkeypatch):
    """AGEMM_EPOCH_BASE = 2^32 - 3 starts the flags' and consumed counts' epochs just below
    their 32-bit wrap (both are compared by wrap-aware differences). After two epochs of
    NaN partials, eight epochs with three data sets, tiles released late and out of
    order, take every count across the wrap. Each output must match its own partials: the
    rank-order BSP result of a context counting from zero, within the tolerance (the
    fused combine folds ranks in arrival order)."""
    import torch
    W, H, D, HT = 8, 96, 128, 16
    sets = [synth.fd_partials(0x7800 + 16 * k, W, H, D) for k in range(3)]
    devs = [_dev_parts(o, l) for o, l in sets]
    plain = _ctx(W, H, D, HT, "f32")
    refs = []
    for k in range(3):
        O = _out(H, D, "f32")
        plain.run_bsp(*devs[k], O)
        refs.append(O)
    torch.cuda.synchronize()
    plain.check()
    assert np.abs(refs[0].cpu().numpy().astype(np.float64) - fdo.combine(*sets[0])).max() <= fdo.tolerance("f32")
    from shard_decomposed_gemm_amd import AgemmError
    from shard_decomposed_gemm_amd.agemm import EINVAL
    monkeypatch.setenv("AGEMM_EPOCH_BASE", "0x1ffffffff")  # past 32 bits: refused, so the hook is read
    with pytest.raises(AgemmError) as ei:
        _ctx(W, H, D, HT, "f32")
    assert ei.value.status == EINVAL
    monkeypatch.setenv("AGEMM_EPOCH_BASE", str(2**32 - 3))
    ctx = _ctx(W, H, D, HT, "f32")
    sp, sc = ctx.streams()
    nan_o = [torch.full((H, D), float("nan"), dtype=torch.float32, device=gu.dev()) for _ in range(W)]
    nan_l = [torch.full((H,), float("nan"), dtype=torch.float32, device=gu.dev()) for _ in range(W)]
    ctx.produce(nan_o, nan_l, stream=sp)
    ctx.produce(nan_o, nan_l, stream=sp)
    outs = []
    for e in range(8):
        k = e % 3
        order, offs = synth.schedule(0x7900 + e, ctx.t, 3_000)
        O = _out(H, D, "f32")
        ctx.produce(*devs[k], schedule=(order, offs), stream=sp)
        ctx.run_fused(O, stream=sc)
        outs.append(O)
    torch.cuda.synchronize()
    ctx.check()
    for e, O in enumerate(outs):
        assert np.abs(O.cpu().numpy().astype(np.float64) - refs[e % 3].cpu().numpy().astype(np.float64)).max() \
            <= fdo.tolerance("f32"), e


def test_fd_inbox_guard_holds_the_producer_for_a_late_combine():
    """The combine of epoch 0 starts late (its stream first runs a spin kernel of tens of
    milliseconds), after the producers of epochs 1 and 2 were issued. Epoch 2 reuses epoch 0's inbox:
    its producer must wait on the device until that combine has read it (timed: it
    spans most of the spin), so every epoch's output still matches its own partials."""
    import torch
    W, H, D, HT = 8, 96, 128, 16
    sets = [synth.fd_partials(0x7B00 + 16 * k, W, H, D) for k in range(3)]
    refs = [fdo.combine(o, l) for o, l in sets]
    devs = [_dev_parts(o, l) for o, l in sets]
    ctx = _ctx(W, H, D, HT, "f32")
    sp, sc = ctx.streams()
    torch.cuda.synchronize()
    h0, h1 = gu.hold_stream(sc, 40.0)
    p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    outs = []
    for k in range(3):
        O = _out(H, D, "f32")
        if k == 2:
            p0.record(sp)
        ctx.produce(*devs[k], stream=sp)
        if k == 2:
            p1.record(sp)
        ctx.run_fused(O, stream=sc)
        outs.append(O)
    torch.cuda.synchronize()
    ctx.check()
    held, waited = h0.elapsed_time(h1), p0.elapsed_time(p1)
    assert held > 15.0, held
    assert waited > 0.5 * held, (waited, held)
    for k, O in enumerate(outs):
        assert np.abs(O.cpu().numpy().astype(np.float64) - refs[k]).max() <= fdo.tolerance("f32"), k


def test_fd_timeout_reports_and_recovers():
    """A tile released long after the spin timeout: the combine stops waiting, fdc_check
    reports ETIMEOUT, and the next epoch is correct again."""
    import torch
    from shard_decomposed_gemm_amd import AgemmError
    from shard_decomposed_gemm_amd.agemm import ETIMEOUT
    W, H, D, HT = 8, 32, 128, 16
    o, lse = synth.fd_partials(0x7800, W, H, D)
    ref = fdo.combine(o, lse)
    do, dl = _dev_parts(o, lse)
    ctx = _ctx(W, H, D, HT, "f32")
    ctx.set_spin_timeout_us(2_000)
    order = np.arange(ctx.t, dtype=np.int32)
    offs = np.zeros(ctx.t, dtype=np.int64)
    offs[-1] = 30_000_000  # last tile 30 ms late
    # the context's stream pair runs the combine concurrently with the producer
    sp, sc = ctx.streams()
    O = _out(H, D, "f32")
    ctx.produce(do, dl, schedule=(order, offs), stream=sp)
    ctx.run_fused(O, stream=sc)
    torch.cuda.synchronize()
    with pytest.raises(AgemmError) as ei:
        ctx.check()
    assert ei.value.status == ETIMEOUT
    ctx.check()
    ctx.set_spin_timeout_us(2_000_000)
    O2 = _out(H, D, "f32")
    ctx.produce(do, dl, stream=sp)
    ctx.run_fused(O2, stream=sc)
    torch.cuda.synchronize()
    ctx.check()
    assert np.abs(O2.cpu().numpy().astype(np.float64) - ref).max() <= fdo.tolerance("f32")


def test_fd_call_order_and_argument_errors():
    import torch
    from shard_decomposed_gemm_amd import AgemmError
    from shard_decomposed_gemm_amd.agemm import EINVAL, ESTATE
    W, H, D, HT = 4, 32, 64, 8
    o, lse = synth.fd_partials(0x7900, W, H, D)
    do, dl = _dev_parts(o, lse)
    ctx = _ctx(W, H, D, HT, "f16")
    O = _out(H, D, "f16")
    with pytest.raises(AgemmError) as ei:
        ctx.run_fused(O)
    assert ei.value.status == ESTATE
    dup = (np.zeros(ctx.t, dtype=np.int32), np.zeros(ctx.t, dtype=np.int64))
    with pytest.raises(AgemmError) as ei:
        ctx.produce(do, dl, schedule=dup)
    assert ei.value.status == EINVAL
    with pytest.raises(ValueError):
        ctx.produce(do[:-1], dl[:-1])
    torch.cuda.synchronize()
