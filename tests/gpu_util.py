"""Shared input plumbing for the GPU tests (no arithmetic of the method)."""
from __future__ import annotations

import numpy as np

import synth


def dev():
    import torch
    return torch.device("cuda:0")


def to_dev(bits: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.float16)).to(dev())


def random_problem(W, M, K, N, seed=1):
    """fp16 uniform[-1, 1] inputs from the shared generator (bits on host, tensors on device)."""
    a = synth.matrix_f16(0xA000 + seed, M, K)
    b = synth.matrix_f16(0xB000 + seed, K, N)
    sh = synth.shards(a, W)
    return a, sh, b, [to_dev(s) for s in sh], to_dev(b)


def coarse_bits(seed, rows, cols, levels=16):
    """fp16 values j/levels, |j| <= levels: every product and partial sum is exact in fp32,
    so a correct GPU result equals the oracle bit for bit whatever the summation order."""
    u = synth.fill_f16(seed, rows * cols).view(np.float16).astype(np.float64)
    q = np.rint(u * levels) / levels
    return q.astype(np.float16).view(np.uint16).reshape(rows, cols)


def empty_c(M, N, c_dtype):
    import torch
    dt = torch.float16 if c_dtype == "f16" else torch.float32
    return torch.full((M, N), float("nan"), dtype=dt, device=dev())


def c_to_f64(C) -> np.ndarray:
    return C.float().cpu().numpy().astype(np.float64)


def pick_consumer(monkeypatch, kernel):
    """Selects the consumer of contexts created afterwards: "small_m" lets the small-M
    streaming kernel take M up to 8 (by default it runs at M = 1 only), "mfma" keeps it
    off at every M, None leaves the default choice."""
    if kernel == "small_m":
        monkeypatch.setenv("AGEMM_SMALL_M_MAX", "8")
    elif kernel == "mfma":
        monkeypatch.setenv("AGEMM_SMALL_M_MAX", "0")
    elif kernel is not None:
        raise ValueError(kernel)


def assert_consumer(ctx, kernel):
    if kernel is not None:
        assert ctx.consumer_info()["kind"] == kernel, ctx.consumer_info()


def hold_stream(stream, ms: float):
    """Queues on `stream` a one-wave spin kernel (torch.cuda._sleep) that delays the
    stream's later work by at least `ms` milliseconds without occupying the CUs: it
    spins for ms x 2.4e6 engine-clock cycles, and the part's engine clock never exceeds
    2.4 GHz (at a lower clock the hold is longer). Returns timing events around it."""
    import torch
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        start.record()
        torch.cuda._sleep(int(ms * 2.4e6))
        end.record()
    return start, end
