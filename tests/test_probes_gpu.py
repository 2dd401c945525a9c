"""The measurement probes the bench reports (MFMA-only ceiling, global->LDS tile-load throughput) launch on the GPU
and return figures inside the physical limits of the part."""
import pytest

from implicit_gemm_conv_amd import probes

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("mfma,waves", [(16, 8), (32, 8), (16, 4), (32, 4)])
def test_mfma_ceiling(mfma, waves):
    r = probes.mfma_ceiling(mfma, waves, iters=1000, grid=256, reps=2)
    assert 0.3 < r["ghz"] < 2.6, r
    # never above the spec peak at the clock it ran at (a few % for clock-reading granularity)
    assert 0.2 < r["per_clock_frac"] <= 1.03, r
    assert r["tflops"] <= probes.PEAK_BF16_TFLOPS * 1.03, r


@pytest.mark.parametrize("bk", [16, 32, 64])
def test_dma_throughput(bk):
    r = probes.dma_throughput(bk, 3, reps=2)
    assert 0.3 < r["ghz"] < 2.6, r
    # a CU's vector memory path moves at most 128 bytes per clock
    assert 1.0 < r["B/clk/CU"] <= 128, r
