"""The MFMA consumer's work plan (host logic, no GPU): tile configuration, grid and
whether the stream-K split is used, through agemm_mfma_plan."""
import itertools

import pytest

from shard_decomposed_gemm_amd import agemm

CUS = 256  # MI355X compute units


def _tiles(M, N, cfg):
    bm = 128 if cfg == 1 else 256
    bn = 256 if cfg == 0 else 128
    return -(-M // bm) * -(-N // bn)


def _default_cfg(M):
    return 1 if M <= 128 else 2 if M <= 256 else 0


@pytest.mark.parametrize("M,N,cfg,grid,split", [
    (128, 28672, 1, 224, False),   # crossover workload: 224 whole 128x128 tiles (split loses here)
    (256, 28672, 2, 224, False),   # one row block of 256x128 tiles
    (129, 28672, 2, 224, False),
    (257, 28672, 0, 224, False),
    (512, 28672, 0, 224, False),   # out-of-order workload: 224 whole 256x256 tiles
    (4096, 28672, 0, 256, False),  # prefill workload: 1792 tiles, 7 per CU
    (128, 4096, 1, 256, True),     # 32 tiles: split over one workgroup per CU
    (512, 2048, 0, 128, True),     # 16 tiles x 8 shards = 128 units
    (512, 8192, 0, 224, True),     # 64 tiles x 8 shards over 7/8 of the CUs: the 256-row split
                                   # kernel leaves no room beside it for producer waves
    (9, 256, 1, 16, True),         # 2 tiles x 8 shards
])
def test_workload_plans(M, N, cfg, grid, split):
    """The plans at the workloads' K = 8192, W = 8."""
    assert agemm.mfma_plan(M, N, 8192, 8, CUS) == (cfg, grid, split)


@pytest.mark.parametrize("M,N,K,split", [
    (8, 256, 2048, False),     # 2 tiles: the split would save 7 x 256 columns
    (8, 256, 4096, False),     # 7 x 512 = 3584 columns
    (8, 256, 8192, True),      # 7 x 1024
    (128, 4096, 4096, False),  # 32 tiles
    (128, 4096, 8192, True),
    (300, 1032, 4096, False),  # 10 tiles of 256x256
    (300, 1032, 8192, True),
    (8, 256, 512, False),      # the tiny workload
])
def test_split_needs_enough_k(M, N, K, split):
    """The automatic split also needs to save the busiest workgroup at least 4096 columns
    of K: below that its hand-off costs more than the shorter run (measured crossovers)."""
    assert agemm.mfma_plan(M, N, K, 8, CUS)[2] == split
    assert agemm.mfma_plan(M, N, K, 8, CUS, split_mode=1)[2] is True


def test_forced_modes_and_single_shard():
    assert agemm.mfma_plan(128, 28672, 8192, 8, CUS, split_mode=1) == (1, 256, True)
    assert agemm.mfma_plan(128, 4096, 8192, 8, CUS, split_mode=0) == (1, 32, False)
    for mode in (-1, 0, 1):  # one shard: nothing to split
        assert agemm.mfma_plan(128, 1024, 8192, 1, CUS, split_mode=mode)[2] is False
    assert agemm.mfma_plan(300, 1000, 8192, 8, CUS, tile_config=1)[0] == 1
    assert agemm.mfma_plan(100, 1000, 8192, 8, CUS, tile_config=0)[0] == 0
    assert agemm.mfma_plan(100, 1000, 8192, 8, CUS, tile_config=2)[0] == 2


def test_plan_invariants_over_a_sweep():
    for M, N, W, KS, cus, tc, mode in itertools.product((1, 9, 128, 129, 256, 300, 4096), (8, 264, 4096, 28672),
                                                        (1, 2, 3, 8, 16), (64, 512, 4096), (7, 80, 256, 304),
                                                        (-1, 0, 1, 2), (-1, 0, 1)):
        cfg, grid, split = agemm.mfma_plan(M, N, W * KS, W, cus, tc, mode)
        assert cfg == (tc if tc >= 0 else _default_cfg(M))
        t = _tiles(M, N, cfg)
        if split:
            # the 256-row tiles' split kernels leave an eighth of the CUs to the producer
            assert W >= 2 and grid == min(t * W, cus if cfg == 1 else max(1, cus - cus // 8))
            if mode == -1:  # automatic: half of the CUs idle and 4096 columns of K saved
                run_tiles = -(-t // min(t, cus)) * W
                scus = cus if cfg == 1 else max(1, cus - cus // 8)
                run_units = -(-(t * W) // min(t * W, scus))
                assert 2 * t <= cus and (run_tiles - run_units) * KS >= 4096
        else:
            assert grid == min(t, cus)
        assert 1 <= grid <= cus


@pytest.mark.parametrize("args", [(0, 64, 512, 8, CUS, -1, -1), (8, 4, 512, 8, CUS, -1, -1),
                                  (8, 64, 512, 0, CUS, -1, -1), (8, 64, 512, 17, CUS, -1, -1),
                                  (8, 64, 512, 8, 0, -1, -1), (8, 64, 512, 8, CUS, 3, -1),
                                  (8, 64, 512, 8, CUS, -1, 2), (8, 64, 100, 8, CUS, -1, -1),
                                  (8, 64, 4, 8, CUS, -1, -1)])
def test_plan_rejects_bad_arguments(args):
    with pytest.raises(agemm.AgemmError) as ei:
        agemm.mfma_plan(*args)
    assert ei.value.status == agemm.EINVAL
