"""The bench's measurement aids (libswiglu_probe.so): the plain streaming
read and the device attributes."""
import pytest

pytestmark = pytest.mark.gpu


def test_device_record_is_mi355x():
    import bench
    d = bench.device_record()
    assert d.get("compute_units") == 256, d
    assert d["max_clock_mhz"] == pytest.approx(2400.0, rel=0.01), d
    assert d["bf16_peak_tflops"] == pytest.approx(bench.BF16_PEAK_TFLOPS, rel=0.01), d


def test_read_ceiling_is_a_plausible_hbm_rate():
    import bench
    rc = bench.read_ceiling(256 << 20)
    assert rc["bytes"] == 256 << 20
    # a plain read of 256 MiB from HBM: well above half and below the 8 TB/s peak
    assert 4000.0 < rc["gbps"] < bench.HBM_PEAK_GBS, rc
    assert bench.read_ceiling(256 << 20) is rc   # cached per size
