"""Flag gating on the GPU: the consumer never reads a k-tile before its flag.

Source of the invariant: "Eliminating Multi-GPU Performance Taxes" analysis
page, correctness check #4 (the store precedes the flag increment, so a
consumer that sees the flag sees the data).
"""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _ctx(W, M, K, N, c_dtype="f16"):
    from shard_decomposed_gemm_amd import Context
    return Context(W, M, K, N, c_dtype=c_dtype)


@pytest.fixture(params=["relaxed", "strict"])
def gate_mode(request, monkeypatch):
    """Both consumer gate modes: fence-free (default) and the formal agent-scope acquire."""
    monkeypatch.setenv("AGEMM_STRICT_ACQUIRE", "1" if request.param == "strict" else "0")
    return request.param


@pytest.mark.parametrize("W,M,K,N,kernel", [
    (8, 1, 2048, 1024, "small_m"), (8, 1, 2048, 1024, "mfma"),
    (8, 4, 4096, 2056, "small_m"), (8, 4, 4096, 2056, "mfma"),
    (8, 96, 2048, 1024, "mfma"), (8, 512, 2048, 1024, "mfma"),
])
def test_poisoned_inbox_is_never_read_early(W, M, K, N, kernel, gate_mode, monkeypatch):
    """Epochs 1 and 2 fill both inboxes with NaN; epoch 3 releases real tiles late and
    out of order while the consumer is already running. Any premature read would show NaN."""
    import torch
    a, sh, b, dsh, B = gu.random_problem(W, M, K, N, seed=41)
    ref = oracle.sharded_gemm(sh, b)
    gu.pick_consumer(monkeypatch, kernel)
    ctx = _ctx(W, M, K, N, "f32")
    gu.assert_consumer(ctx, kernel)
    nan = [torch.full((M, K // W), float("nan"), dtype=torch.float16, device=gu.dev()) for _ in range(W)]
    ctx.produce(nan)
    ctx.produce(nan)  # epochs alternate between two inboxes: poison both
    torch.cuda.synchronize()
    order, offs = synth.schedule(0x5100 + M, ctx.t, 40_000)  # up to 40 us between releases
    sp, sc = ctx.streams()
    C = gu.empty_c(M, N, "f32")
    ctx.produce(dsh, schedule=(order, offs), stream=sp)
    ctx.run_fused(B, C, stream=sc)
    torch.cuda.synchronize()
    ctx.check()
    got = gu.c_to_f64(C)
    assert np.isfinite(got).all()
    assert np.abs(got - ref).max() <= oracle.tolerance(K)


@pytest.mark.parametrize("W,M,K,N,bkf,kernel", [
    (8, 300, 8192, 1000, 128, None),   # 256x256 MFMA tiles, 8 flag tiles per shard
    (8, 130, 4096, 520, 64, None),     # 128x128 MFMA tiles, one k-step per flag tile
    (8, 4, 4096, 1032, 64, "small_m"), # small-M streaming kernel
    (8, 4, 4096, 1032, 64, "mfma"),    # the same on 128x128 MFMA tiles (the default at M = 4)
    (8, 1, 4096, 1024, 64, "small_m"), # small-M, M = 1
    (16, 257, 16384, 264, 256, None),  # 16 shards of 4 flag tiles
])
def test_sixty_four_flags_out_of_order(W, M, K, N, bkf, kernel, monkeypatch):
    """The largest flag count, T = W * KS / BK_f = 64 (one flag per lane of the polling
    wave), with a non-default flag k-tile: poisoned inboxes, then the 64 tiles released
    in a seeded order with cumulative delays while the consumer runs."""
    import torch
    from shard_decomposed_gemm_amd import Context
    a, sh, b, dsh, B = gu.random_problem(W, M, K, N, seed=43)
    ref = oracle.sharded_gemm(sh, b)
    gu.pick_consumer(monkeypatch, kernel)
    ctx = Context(W, M, K, N, c_dtype="f32", flag_ktile=bkf)
    gu.assert_consumer(ctx, kernel)
    assert ctx.t == 64
    nan = [torch.full((M, K // W), float("nan"), dtype=torch.float16, device=gu.dev()) for _ in range(W)]
    ctx.produce(nan)
    ctx.produce(nan)
    torch.cuda.synchronize()
    order, offs = synth.schedule(0x5300 + M, ctx.t, 10_000)
    sp, sc = ctx.streams()
    C = gu.empty_c(M, N, "f32")
    ctx.produce(dsh, schedule=(order, offs), stream=sp)
    ctx.run_fused(B, C, stream=sc)
    torch.cuda.synchronize()
    ctx.check()
    got = gu.c_to_f64(C)
    assert np.isfinite(got).all()
    assert np.abs(got - ref).max() <= oracle.tolerance(K)


@pytest.mark.parametrize("M", [1, 256])
def test_alternating_epochs(M, gate_mode):
    """Three data sets cycle over successive epochs on two streams (so each of the two
    inboxes holds a different data set every time it is reused); each epoch's C must
    match its own data (an inbox is not overwritten while still being read)."""
    import torch
    W, K, N = 8, 2048, 1024
    probs = [gu.random_problem(W, M, K, N, seed=s) for s in (51, 52, 53)]
    refs = [oracle.sharded_gemm(p[1], p[2]) for p in probs]
    ctx = _ctx(W, M, K, N, "f32")
    sp, sc = ctx.streams()
    outs = []
    for e in range(6):
        p = probs[e % 3]
        C = gu.empty_c(M, N, "f32")
        order, offs = synth.schedule(0x5200 + e, ctx.t, 5_000 if e % 3 == 0 else 0)
        ctx.produce(p[3], schedule=(order, offs), stream=sp)
        ctx.run_fused(p[4], C, stream=sc)
        outs.append(C)
    torch.cuda.synchronize()
    ctx.check()
    for e, C in enumerate(outs):
        assert np.abs(gu.c_to_f64(C) - refs[e % 3]).max() <= oracle.tolerance(K), e


@pytest.mark.parametrize("M", [1, 130, 512])
def test_epochs_across_the_flag_counter_wrap(M, monkeypatch):
    """The flags are 32-bit counters, compared with each epoch's target by a wrap-aware
    difference. AGEMM_EPOCH_BASE = 2^32 - 3 starts both inboxes' epoch counts just below
    the wrap, so that the calls after two poisoning ones take every flag and target
    across it. Each epoch's C (three data sets cycling, tiles released late and out of
    order into inboxes that held NaN or another data set) must equal its own Pull result
    bit for bit."""
    import torch
    from shard_decomposed_gemm_amd import AgemmError
    from shard_decomposed_gemm_amd.agemm import EINVAL
    W, K, N = 8, 2048, 1544
    for bad in ("4294967296", "-1", "base"):  # the hook is read: values it cannot take are refused
        monkeypatch.setenv("AGEMM_EPOCH_BASE", bad)
        with pytest.raises(AgemmError) as ei:
            _ctx(W, M, K, N, "f16")
        assert ei.value.status == EINVAL, bad
    monkeypatch.setenv("AGEMM_EPOCH_BASE", str(2**32 - 3))
    probs = [gu.random_problem(W, M, K, N, seed=s) for s in (91, 92, 93)]
    ctx = _ctx(W, M, K, N, "f16")
    refs = []
    for p in probs:
        C = gu.empty_c(M, N, "f16")
        ctx.run_pull(p[3], p[4], C)
        refs.append(C)
    torch.cuda.synchronize()
    assert np.abs(gu.c_to_f64(refs[0]) - oracle.sharded_gemm(probs[0][1], probs[0][2])).max() <= oracle.tolerance(K)
    sp, sc = ctx.streams()
    nan = [torch.full((M, K // W), float("nan"), dtype=torch.float16, device=gu.dev()) for _ in range(W)]
    ctx.produce(nan, stream=sp)
    ctx.produce(nan, stream=sp)
    outs = []
    for e in range(8):  # epoch counts 2^32 - 1, 0, 1, 2 on each inbox
        p = probs[e % 3]
        order, offs = synth.schedule(0x5400 + e, ctx.t, 10_000)
        C = gu.empty_c(M, N, "f16")
        ctx.produce(p[3], schedule=(order, offs), stream=sp)
        ctx.run_fused(p[4], C, stream=sc)
        outs.append(C)
    torch.cuda.synchronize()
    ctx.check()
    for e, C in enumerate(outs):
        assert torch.equal(C.view(torch.int16), refs[e % 3].view(torch.int16)), e
    ctx.close()


@pytest.mark.parametrize("M", [1, 2, 300])
def test_timeout_reports_and_recovers(M):
    """A tile released long after the consumer's spin timeout: the consumer stops,
    agemm_check reports ETIMEOUT, and the next epoch is correct again."""
    import torch
    from shard_decomposed_gemm_amd import AgemmError
    from shard_decomposed_gemm_amd.agemm import ETIMEOUT
    W, K, N = 8, 2048, 1024
    a, sh, b, dsh, B = gu.random_problem(W, M, K, N, seed=61)
    ref = oracle.sharded_gemm(sh, b)
    ctx = _ctx(W, M, K, N, "f32")
    ctx.set_spin_timeout_us(2_000)
    order = np.arange(ctx.t, dtype=np.int32)
    offs = np.zeros(ctx.t, dtype=np.int64)
    offs[-1] = 30_000_000  # last tile 30 ms late
    # the context's stream pair runs the consumer concurrently with the producer, so
    # the consumer is waiting when the late tile's deadline passes
    sp, sc = ctx.streams()
    C = gu.empty_c(M, N, "f32")
    ctx.produce(dsh, schedule=(order, offs), stream=sp)
    ctx.run_fused(B, C, stream=sc)
    torch.cuda.synchronize()
    with pytest.raises(AgemmError) as ei:
        ctx.check()
    assert ei.value.status == ETIMEOUT
    ctx.check()  # the error word is cleared
    ctx.set_spin_timeout_us(2_000_000)
    C2 = gu.empty_c(M, N, "f32")
    ctx.produce(dsh, stream=sp)
    ctx.run_fused(B, C2, stream=sc)
    torch.cuda.synchronize()
    ctx.check()
    assert np.abs(gu.c_to_f64(C2) - ref).max() <= oracle.tolerance(K)


@pytest.mark.parametrize("M,kernel", [(1, "small_m"), (130, "mfma"), (4, "mfma"), (1040, "mfma")])
def test_inbox_guard_holds_the_producer_for_a_late_consumer(M, kernel):
    """The producer waits on the device until the fused consumers that read its
    inbox before are done with it (both consumer kernels count themselves out of
    the inbox); above M = 1024 its stream also waits for the last of them. The
    consumer of the first epoch starts late (its stream first runs a spin kernel of
    tens of milliseconds), after the producers of the next two epochs were issued;
    the third epoch reuses the first one's inbox, so its producer must hold until
    that consumer has read it (timed: it spans most of the spin). Every epoch's C
    must equal its own Pull result bit for bit."""
    import torch
    W, K, N = 8, 2048, 1544
    probs = [gu.random_problem(W, M, K, N, seed=s) for s in (71, 72, 73)]
    ctx = _ctx(W, M, K, N, "f16")
    gu.assert_consumer(ctx, kernel)
    refs = []
    for p in probs:
        C = gu.empty_c(M, N, "f16")
        ctx.run_pull(p[3], p[4], C)
        refs.append(C)
    torch.cuda.synchronize()
    sp, sc = ctx.streams()
    h0, h1 = gu.hold_stream(sc, 40.0)
    p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    outs = []
    for e in range(3):
        C = gu.empty_c(M, N, "f16")
        if e == 2:
            p0.record(sp)
        ctx.produce(probs[e][3], stream=sp)
        if e == 2:
            p1.record(sp)
        ctx.run_fused(probs[e][4], C, stream=sc)
        outs.append(C)
    torch.cuda.synchronize()
    ctx.check()
    held, waited = h0.elapsed_time(h1), p0.elapsed_time(p1)
    assert held > 15.0, held  # the consumer really started late
    assert waited > 0.5 * held, (waited, held)  # and the producer held for it
    for e, C in enumerate(outs):
        assert torch.equal(C.view(torch.int16), refs[e].view(torch.int16)), e
    ctx.close()


@pytest.mark.parametrize("M,kernel", [(1, "small_m"), (130, "mfma")])
def test_inbox_guard_timeout_reports_and_recovers(M, kernel):
    """The consumer of the first epoch is held (a spin kernel of tens of milliseconds on
    its stream) for longer than the 2 ms spin timeout, so the producer of the third epoch (same inbox)
    gives up waiting: agemm_check reports ETIMEOUT for the producer, and later epochs are
    correct again."""
    import torch
    from shard_decomposed_gemm_amd import AgemmError
    from shard_decomposed_gemm_amd.agemm import ETIMEOUT
    W, K, N = 8, 2048, 1024
    a, sh, b, dsh, B = gu.random_problem(W, M, K, N, seed=62)
    ref = oracle.sharded_gemm(sh, b)
    ctx = _ctx(W, M, K, N, "f32")
    gu.assert_consumer(ctx, kernel)
    sp, sc = ctx.streams()
    ctx.set_spin_timeout_us(2_000)
    h0, h1 = gu.hold_stream(sc, 40.0)
    late = [gu.empty_c(M, N, "f32") for _ in range(3)]  # kept alive until the kernels have run
    for C in late:
        ctx.produce(dsh, stream=sp)
        ctx.run_fused(B, C, stream=sc)
    torch.cuda.synchronize()
    assert h0.elapsed_time(h1) > 15.0
    with pytest.raises(AgemmError) as ei:
        ctx.check()
    assert ei.value.status == ETIMEOUT
    assert "producer" in str(ei.value)
    ctx.check()  # the error word is cleared
    ctx.set_spin_timeout_us(2_000_000)
    outs = []
    for e in range(3):
        C = gu.empty_c(M, N, "f32")
        ctx.produce(dsh, stream=sp)
        ctx.run_fused(B, C, stream=sc)
        outs.append(C)
    torch.cuda.synchronize()
    ctx.check()
    for C in outs:
        assert np.abs(gu.c_to_f64(C) - ref).max() <= oracle.tolerance(K)
    ctx.close()


@pytest.mark.parametrize("M", [1, 130])
def test_producer_order_survives_a_switch_from_the_context_streams(M):
    """Producer events on the context's own streams are recorded only when a call on
    another stream needs them. The first producer runs on the context's producer stream
    behind a spin kernel of tens of milliseconds; the next two run on the default stream
    and must still come after it. The third reuses the first one's inbox: had it
    overtaken the first, its consumer would read the first epoch's data."""
    import torch
    W, K, N = 8, 2048, 1544
    probs = [gu.random_problem(W, M, K, N, seed=s) for s in (81, 82, 83)]
    ctx = _ctx(W, M, K, N, "f16")
    refs = []
    for p in probs:
        C = gu.empty_c(M, N, "f16")
        ctx.run_pull(p[3], p[4], C)
        refs.append(C)
    torch.cuda.synchronize()
    sp, sc = ctx.streams()
    h0, h1 = gu.hold_stream(sp, 40.0)
    ctx.produce(probs[0][3], stream=sp)
    ctx.produce(probs[1][3])  # default stream
    p2 = torch.cuda.Event(enable_timing=True)
    p2.record()
    ctx.produce(probs[2][3])
    C = gu.empty_c(M, N, "f16")
    ctx.run_fused(probs[2][4], C)
    torch.cuda.synchronize()
    ctx.check()
    assert h0.elapsed_time(h1) > 15.0
    assert h0.elapsed_time(p2) >= h0.elapsed_time(h1)  # the second producer ran after the held one
    assert torch.equal(C.view(torch.int16), refs[2].view(torch.int16))
    ctx.close()


@pytest.mark.parametrize("M", [1, 130])
def test_consumer_order_survives_a_switch_from_the_context_streams(M):
    """Consumer events on the context's own streams are recorded only when a call on
    another stream needs them. A fused consumer on the context's consumer stream waits
    behind a spin kernel; a Pull call on the default stream, which shares the context's
    workspaces, must still run after it, and both results stay exact."""
    import torch
    W, K, N = 8, 2048, 1544
    probs = [gu.random_problem(W, M, K, N, seed=s) for s in (84, 85)]
    ctx = _ctx(W, M, K, N, "f16")
    refs = []
    for p in probs:
        C = gu.empty_c(M, N, "f16")
        ctx.run_pull(p[3], p[4], C)
        refs.append(C)
    torch.cuda.synchronize()
    sp, sc = ctx.streams()
    ctx.produce(probs[0][3], stream=sp)
    h0, h1 = gu.hold_stream(sc, 40.0)
    C1 = gu.empty_c(M, N, "f16")
    ctx.run_fused(probs[0][4], C1, stream=sc)
    C2 = gu.empty_c(M, N, "f16")
    ctx.run_pull(probs[1][3], probs[1][4], C2)  # default stream
    q = torch.cuda.Event(enable_timing=True)
    q.record()
    torch.cuda.synchronize()
    ctx.check()
    assert h0.elapsed_time(h1) > 15.0
    assert h0.elapsed_time(q) >= h0.elapsed_time(h1)  # the Pull ran after the held consumer
    assert torch.equal(C1.view(torch.int16), refs[0].view(torch.int16))
    assert torch.equal(C2.view(torch.int16), refs[1].view(torch.int16))
    ctx.close()


def test_call_order_and_argument_errors():
    import torch
    from shard_decomposed_gemm_amd import AgemmError
    from shard_decomposed_gemm_amd.agemm import EINVAL, ESTATE
    W, M, K, N = 8, 16, 1024, 256
    a, sh, b, dsh, B = gu.random_problem(W, M, K, N, seed=71)
    ctx = _ctx(W, M, K, N, "f16")
    C = gu.empty_c(M, N, "f16")
    with pytest.raises(AgemmError) as ei:
        ctx.run_fused(B, C)
    assert ei.value.status == ESTATE
    bad = (np.arange(ctx.t)[::-1].copy(), np.array([5] + [0] * (ctx.t - 1)))  # offsets decrease
    with pytest.raises(AgemmError) as ei:
        ctx.produce(dsh, schedule=bad)
    assert ei.value.status == EINVAL
    dup = (np.zeros(ctx.t, dtype=np.int32), np.zeros(ctx.t, dtype=np.int64))  # not a permutation
    with pytest.raises(AgemmError) as ei:
        ctx.produce(dsh, schedule=dup)
    assert ei.value.status == EINVAL
    # a misaligned C (2-byte offset) is rejected before any launch
    big = torch.empty(M * N + 1, dtype=torch.float16, device=gu.dev())
    ctx.produce(dsh)
    with pytest.raises(AgemmError) as ei:
        import ctypes
        from shard_decomposed_gemm_amd import agemm
        rc = agemm.load().agemm_run_fused(ctx._h, B.data_ptr(), big.data_ptr() + 2, None)
        ctx._raise(rc, "agemm_run_fused")
    assert ei.value.status == EINVAL
    torch.cuda.synchronize()


@pytest.mark.parametrize("split", ["0", "1"])
def test_flag_tiles_above_31_wait_when_tile_31_is_up(split, monkeypatch):
    """T = 64 flags: tiles 0..31 (tile 31 first) are released at once, tiles 32..63 two
    milliseconds later, into poisoned inboxes. A wave's 64-bit record of raised flags
    must not carry bit 31 into bits 32..63 (a sign-extended low half would mark every
    later tile raised and read them before their data). Whole tiles and the stream-K
    split, which starts workgroups at shards 4..7 (tiles 32..63)."""
    import torch
    from shard_decomposed_gemm_amd import Context
    monkeypatch.setenv("AGEMM_SPLIT", split)
    W, M, K, N, bkf = 8, 300, 8192, 1000, 128
    a, sh, b, dsh, B = gu.random_problem(W, M, K, N, seed=47)
    ref = oracle.sharded_gemm(sh, b)
    ctx = Context(W, M, K, N, c_dtype="f32", flag_ktile=bkf)
    assert ctx.t == 64 and ctx.split is (split == "1")
    order = np.array([31] + list(range(31)) + list(range(32, 64)), dtype=np.int32)
    offs = np.array([0] * 32 + [2_000_000 + 1_000 * i for i in range(32)], dtype=np.int64)
    nan = [torch.full((M, K // W), float("nan"), dtype=torch.float16, device=gu.dev()) for _ in range(W)]
    sp, sc = ctx.streams()
    for _ in range(3):
        ctx.produce(nan)
        ctx.produce(nan)
        torch.cuda.synchronize()
        C = gu.empty_c(M, N, "f32")
        ctx.produce(dsh, schedule=(order, offs), stream=sp)
        ctx.run_fused(B, C, stream=sc)
        torch.cuda.synchronize()
        ctx.check()
        got = gu.c_to_f64(C)
        assert np.isfinite(got).all()
        assert np.abs(got - ref).max() <= oracle.tolerance(K)
    ctx.close()


@pytest.mark.parametrize("M,epochs,kernel", [(1, 120, None), (7, 120, "small_m"), (7, 120, "mfma"), (300, 120, None),
                                            (1024, 120, None), (512, 1000, None)])
def test_epoch_stress_bitwise(M, epochs, kernel, gate_mode, monkeypatch):
    """120 (at M = 512: 1000) epochs cycle three data sets with jittered release schedules while the
    consumer runs concurrently. Each epoch's C must equal, bit for bit, the ungated
    (pull) result of its own data set: a read of an inbox's previous content (another
    data set, since three sets cycle over two inboxes) would change it."""
    import torch
    W, K, N = 8, 2048, 1544
    probs = [gu.random_problem(W, M, K, N, seed=s) for s in (81, 82, 83)]
    gu.pick_consumer(monkeypatch, kernel)
    ctx = _ctx(W, M, K, N, "f16")
    gu.assert_consumer(ctx, kernel)
    refs = []
    for p in probs:
        C = gu.empty_c(M, N, "f16")
        ctx.run_pull(p[3], p[4], C)
        refs.append(C)
    torch.cuda.synchronize()
    ref0 = oracle.sharded_gemm(probs[0][1], probs[0][2])
    assert np.abs(gu.c_to_f64(refs[0]) - ref0).max() <= oracle.tolerance(K)
    sp, sc = ctx.streams()
    outs = [gu.empty_c(M, N, "f16") for _ in range(4)]
    bad = []
    for e in range(epochs):
        p = probs[e % 3]
        order, offs = synth.schedule(0x5300 + e, ctx.t, (e % 5) * 3_000)
        C = outs[e % 4]
        ctx.produce(p[3], schedule=(order, offs), stream=sp)
        ctx.run_fused(p[4], C, stream=sc)
        if e % 4 == 3:
            torch.cuda.synchronize()
            for j in range(4):
                if not torch.equal(outs[j].view(torch.int16), refs[(e - 3 + j) % 3].view(torch.int16)):
                    bad.append(e - 3 + j)
    torch.cuda.synchronize()
    ctx.check()
    assert not bad, f"epochs with a result different from their own data: {bad}"


def test_stream_pair_runs_producer_and_consumer_concurrently():
    """agemm_streams: the consumer launched second must start while the producer still
    waits to release its last tile (2 ms late), so its own kernel time spans the wait;
    the same pair comes back on later calls."""
    import torch
    W, M, K, N = 8, 300, 2048, 1000
    a, sh, b, dsh, B = gu.random_problem(W, M, K, N, seed=91)
    ctx = _ctx(W, M, K, N, "f32")
    sp, sc = ctx.streams()
    assert ctx.streams() == (sp, sc)
    order = np.arange(ctx.t, dtype=np.int32)
    offs = np.zeros(ctx.t, dtype=np.int64)
    offs[-1] = 2_000_000
    C = gu.empty_c(M, N, "f32")
    ctx.timing_begin(1)
    ctx.produce(dsh, schedule=(order, offs), stream=sp)
    ctx.run_fused(B, C, stream=sc)
    torch.cuda.synchronize()
    (us,) = ctx.timing_end()
    ctx.check()
    assert us >= 1500.0, f"consumer ran {us:.0f} us: it did not overlap the producer"
    assert np.abs(gu.c_to_f64(C) - oracle.sharded_gemm(sh, b)).max() <= oracle.tolerance(K)
    ctx.close()
