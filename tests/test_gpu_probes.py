"""The device ceilings measured beside the published peaks: device properties, a
register-only fp16 MFMA loop and a streaming read. These are calibration figures,
so the checks are ranges a working MI355X lands in, not exact values."""
import pytest

pytestmark = pytest.mark.gpu


def test_device_info():
    from shard_decomposed_gemm_amd import agemm
    info = agemm.device_info()
    assert info["cus"] >= 1 and info["clock_khz"] > 0
    assert info["mem_clock_khz"] > 0 and info["bus_bits"] > 0


def test_mfma_loop_ceiling():
    """Dense fp16 MFMA from registers: above a quarter of the published 2.5 PF and
    not above the peak at the device's own clock (plus 5 % for timing spread)."""
    from shard_decomposed_gemm_amd import agemm
    info = agemm.device_info()
    ceiling = info["cus"] * 4096 * info["clock_khz"] * 1e3 / 1e12
    tf = agemm.probe_mfma(20, 10)
    assert 625.0 < tf <= 1.05 * ceiling, (tf, ceiling)


def test_streaming_read_ceiling():
    """A 1 GiB streaming read (four times the last-level cache): above 2 TB/s and
    below the published 8 TB/s HBM peak plus 5 %."""
    import torch
    from shard_decomposed_gemm_amd import agemm
    buf = torch.zeros(1 << 30, dtype=torch.uint8, device="cuda")
    gbs = agemm.probe_read(buf, 5, 10)
    assert 2000.0 < gbs < 8400.0, gbs
    with pytest.raises(agemm.AgemmError) as ei:
        agemm.probe_read(buf[:15])  # not a multiple of 16 bytes
    assert ei.value.status == agemm.EINVAL
