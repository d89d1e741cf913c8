"""agemm_pull_noalloc (no context, no device allocation) against agemm_run_pull.

Two calls in a row on each path, the second with a smaller input, so that the
second call runs on the scratch array the first one left behind. Inputs on a
1/16 grid make every fp32 partial sum exact, so the two entry points must agree
bit for bit whatever their summation order (the context may take the stream-K
split where the no-allocation call runs whole tiles); uniform[-1, 1] inputs are
held to the parity tolerance 1e-3 * sqrt(K) against the context's result.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

PAIRS = {
    # path: (first shape, second, smaller shape), each (W, M, K, N)
    "small_m": ((8, 1, 8192, 28672), (8, 1, 2048, 4104)),   # split-K workspace in the scratch array
    "mfma": ((8, 300, 2048, 1000), (8, 130, 1024, 520)),    # whole tiles, no workspace
    "mfma_few_rows": ((8, 8, 8192, 28672), (8, 2, 2048, 4104)),  # the MFMA kernel at M <= 8
}


def _inputs(W, M, K, N, exact, seed):
    if exact:
        a = gu.coarse_bits(0xE000 + seed + M, M, K)
        b = gu.coarse_bits(0xE100 + seed + N, K, N)
    else:
        a = synth.matrix_f16(0xE200 + seed + M, M, K)
        b = synth.matrix_f16(0xE300 + seed + N, K, N)
    sh = synth.shards(a, W)
    return [gu.to_dev(x) for x in sh], gu.to_dev(b)


@pytest.mark.parametrize("exact", [True, False])
@pytest.mark.parametrize("c_dtype", ["f32", "f16"])
@pytest.mark.parametrize("path", list(PAIRS))
def test_noalloc_matches_run_pull_on_two_calls(path, c_dtype, exact):
    import torch
    from shard_decomposed_gemm_amd import Context, agemm
    for i, (W, M, K, N) in enumerate(PAIRS[path]):
        print(f"[noalloc] {path} call {i} W={W} M={M} K={K} N={N} c={c_dtype} exact={exact}", flush=True)
        dsh, B = _inputs(W, M, K, N, exact, 7 * i)
        ctx = Context(W, M, K, N, c_dtype=c_dtype)
        assert ctx.consumer[0] == ("mfma" if path.startswith("mfma") else path)
        C_ref = gu.empty_c(M, N, c_dtype)
        ctx.run_pull(dsh, B, C_ref)
        torch.cuda.synchronize()
        ctx.check()
        C = gu.empty_c(M, N, c_dtype)  # NaN: every entry must be written
        rc = agemm.pull_noalloc(dsh, B, C)
        assert rc == agemm.OK, agemm.status_string(rc)
        torch.cuda.synchronize()
        got = gu.c_to_f64(C)
        assert np.isfinite(got).all()
        if exact:
            assert torch.equal(C.view(torch.int32 if c_dtype == "f32" else torch.int16),
                               C_ref.view(torch.int32 if c_dtype == "f32" else torch.int16))
        else:
            err = np.abs(got - gu.c_to_f64(C_ref)).max()
            assert err <= oracle.tolerance(K), err
        ctx.close()


def test_noalloc_rejects_a_workspace_beyond_the_scratch_array():
    """M = 1 row of N = 2,100,000 columns with one shard needs 8.4 MB of partials (one K-range)
    against an 8 MiB array: ESHAPE, and C is left untouched."""
    import torch
    from shard_decomposed_gemm_amd import agemm
    W, M, K, N = 1, 1, 64, 2_100_000
    dsh = [torch.zeros((M, K // W), dtype=torch.float16, device=gu.dev()) for _ in range(W)]
    B = torch.zeros((K, N), dtype=torch.float16, device=gu.dev())
    C = gu.empty_c(M, N, "f32")
    assert agemm.pull_noalloc(dsh, B, C) == agemm.ESHAPE
    torch.cuda.synchronize()
    assert torch.isnan(C).all()
