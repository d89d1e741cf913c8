"""Seeded random shapes through every path, bit for bit against the oracle.

Shapes drawn from a fixed seed: W from 1 to 16 shards (odd counts included),
shard widths KS from 64 to 512 columns, M from 1 to 600 rows (every MFMA
tile, and the small-M streaming kernel: by default at M = 1, and on the
shapes with 1 < M <= 8 once more with it asked for), N from 8 to 1600 columns in steps of 8
(ragged tiles), and a flag k-tile chosen among those that divide KS. Inputs
on a 1/16 grid make every fp32 partial sum exact, so the fused path (tiles
released in a seeded random order with delays, into inboxes full of NaN), the
BSP path and the Pull path must each give the oracle's C bit for bit, as the
AG+GEMM core identity of the "Eliminating Multi-GPU Performance Taxes"
analysis page and its correctness check #3 require of any tiling.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _shapes(n=40, seed=0x5EED):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        W = int(rng.choice([1, 2, 3, 4, 5, 8, 16]))
        KS = 64 * int(rng.integers(1, 9))
        M = int(rng.choice([1, 2, 3, 5, 8])) if len(out) % 4 == 0 else int(rng.integers(9, 601))
        N = 8 * int(rng.integers(1, 201))
        ktiles = [b for b in range(64, KS + 1, 64) if KS % b == 0 and (KS // b) * W <= 64]
        if not ktiles:
            continue
        bkf = int(rng.choice(ktiles))
        out.append((W, M, W * KS, N, bkf))
    return out


SHAPES = _shapes()
CASES = [s + (None,) for s in SHAPES] + [s + ("small_m",) for s in SHAPES if 1 < s[1] <= 8]


@pytest.mark.parametrize("W,M,K,N,bkf,kernel", CASES)
def test_random_shape_every_path_exact(W, M, K, N, bkf, kernel, monkeypatch):
    import torch
    from shard_decomposed_gemm_amd import Context
    print(f"[random-shape] W={W} M={M} K={K} N={N} flag_ktile={bkf} consumer={kernel or 'default'}", flush=True)
    gu.pick_consumer(monkeypatch, kernel)
    a = gu.coarse_bits(0x9000 + M + N, M, K)
    b = gu.coarse_bits(0x9100 + K, K, N)
    sh = synth.shards(a, W)
    ref = oracle.sharded_gemm(sh, b)
    dsh = [gu.to_dev(s) for s in sh]
    B = gu.to_dev(b)
    ctx = Context(W, M, K, N, c_dtype="f32", flag_ktile=bkf)
    gu.assert_consumer(ctx, kernel)
    sp, sc = ctx.streams()
    nan = [torch.full((M, K // W), float("nan"), dtype=torch.float16, device=gu.dev()) for _ in range(W)]
    ctx.produce(nan, stream=sp)
    ctx.produce(nan, stream=sp)
    torch.cuda.synchronize()
    order, offs = synth.schedule(0x9200 + N, ctx.t, 4_000)
    outs = {}
    C = gu.empty_c(M, N, "f32")
    ctx.produce(dsh, schedule=(order, offs), stream=sp)
    ctx.run_fused(B, C, stream=sc)
    outs["fused"] = C
    C = gu.empty_c(M, N, "f32")
    ctx.run_bsp(dsh, B, C, schedule=(order, offs), host_sync=False, stream=sc)
    outs["bsp"] = C
    C = gu.empty_c(M, N, "f32")
    ctx.run_pull(dsh, B, C, stream=sc)
    outs["pull"] = C
    torch.cuda.synchronize()
    ctx.check()
    info = ctx.consumer_info()
    ctx.close()
    for path, C in outs.items():
        got = C.cpu().numpy().astype(np.float64)
        bad = np.argwhere(got != ref)
        assert bad.size == 0, (path, info, bad[:5])
