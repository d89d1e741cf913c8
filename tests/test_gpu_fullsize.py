"""Full-size workloads (K = 8192, N = 28672, W = 8) in the launch configuration the
benchmark times. At M = 1 and M = 128 every entry of C is compared with the
oracle; at M = 512 and M = 4096 (where the binary64 oracle would take minutes)
4096 sampled entries are, and every entry is compared across the fused,
bulk-synchronous and pull paths (same kernels, same summation order, so the
three must agree bit for bit; in arrival order the fused consumer sums the
shards in the order their tiles came up, so it is held to the oracle's
tolerance against the other two instead). The launch each workload runs is
asserted first (agemm_consumer_info), so the comparison covers the kernel the
benchmark times; the same launch shapes are checked entry by entry at a small
K in test_gpu_tiled_parity.py.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

W, K, N = 8, 8192, 28672
CONFIGS = {
    # name: (M, schedule?, flag-tile order of the fused consumer, expected consumer launch on 256 CUs)
    "decode_m1": (1, False, "shard", dict(kind="small_m", ranges=4, tiles=448, grid=448, a_panels=0)),
    "xover_m128": (128, False, "shard", dict(kind="mfma", tile_config=1, tiles=224, grid=224, split=0,
                                             b_nontemporal=1, tiles_per_wg=1, a_panels=1)),
    "prefill_m4096": (4096, False, "shard", dict(kind="mfma", tile_config=0, tiles=1792, grid=256, split=0,
                                                 b_nontemporal=0, tiles_per_wg=7, a_panels=1)),
    "ooo_m512": (512, True, "shard", dict(kind="mfma", tile_config=0, tiles=224, grid=224, split=0,
                                          tiles_per_wg=1, a_panels=1)),
    # the benchmark's --order arrival runs of the two MFMA-bound workloads
    "ooo_m512_arrival": (512, True, "arrival", dict(kind="mfma", tile_config=0, tiles=224, split=0)),
    "prefill_m4096_arrival": (4096, False, "arrival", dict(kind="mfma", tile_config=0, tiles=1792, split=0,
                                                           tiles_per_wg=7)),
}
FULL_ORACLE_MAX_M = 128  # every entry checked against the oracle up to this M


@pytest.fixture(scope="module")
def weight():
    b = synth.matrix_f16(0xB002, K, N)
    return b, gu.to_dev(b)


@pytest.mark.parametrize("name", list(CONFIGS))
def test_full_size(name, weight):
    import torch
    from shard_decomposed_gemm_amd import Context
    from shard_decomposed_gemm_amd import agemm
    M, scheduled, order, expect = CONFIGS[name]
    b, B = weight
    print(f"[fullsize] {name} M={M}", flush=True)
    a = synth.matrix_f16(0xA100 + M, M, K)
    sh = synth.shards(a, W)
    dsh = [gu.to_dev(s) for s in sh]
    ctx = Context(W, M, K, N, c_dtype="f16")
    ctx.set_order(order)
    if agemm.device_info()["cus"] == 256:
        info = ctx.consumer_info()
        for k, v in expect.items():
            assert info[k] == v, (k, info)
    sched = synth.schedule(0x5005, ctx.t, 20_000) if scheduled else None
    sp, sc = ctx.streams()
    Cf = gu.empty_c(M, N, "f16")
    ctx.produce(dsh, schedule=sched, stream=sp)
    ctx.run_fused(B, Cf, stream=sc)
    torch.cuda.synchronize()
    ctx.check()
    Cb = gu.empty_c(M, N, "f16")
    ctx.run_bsp(dsh, B, Cb, schedule=sched, host_sync=True)
    Cp = gu.empty_c(M, N, "f16")
    ctx.run_pull(dsh, B, Cp)
    torch.cuda.synchronize()
    ctx.check()
    assert torch.equal(Cb.view(torch.int16), Cp.view(torch.int16))
    if order == "shard":
        assert torch.equal(Cf.view(torch.int16), Cb.view(torch.int16))
    else:
        diff = (Cf.float() - Cb.float()).abs().max().item()
        assert diff <= oracle.tolerance(K), diff
    got = Cf.float().cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    if M <= FULL_ORACLE_MAX_M:
        ref = oracle.sharded_gemm(sh, b)
        err = np.abs(got - ref).max()
        assert err <= oracle.tolerance(K), err
        ctx.close()
        return
    rng = np.random.default_rng(M)
    n_samp = 4096
    rows = rng.integers(0, M, n_samp)
    cols = rng.integers(0, N, n_samp)
    # always include the corners and the shard-tile boundaries of the grid
    rows[:4] = [0, M - 1, 0, M - 1]
    cols[:4] = [0, 0, N - 1, N - 1]
    ref = oracle.sharded_gemm_entries(sh, b, rows, cols)
    err = np.abs(got[rows, cols] - ref).max()
    assert err <= oracle.tolerance(K), err
    ctx.close()
