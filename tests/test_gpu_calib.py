"""The measured ceilings bench.py reports beside the published peaks: they must
be positive, below the published peaks, and ordered (the passes' inner loop,
with its per-logit VALU work, cannot beat the MFMA chains alone)."""
import pytest

pytestmark = pytest.mark.gpu

PEAK_BF16_TFLOPS = 2516.6
PEAK_HBM_GBS = 8000.0


def test_pass_mix_ceiling_is_ordered_and_below_peak():
    import bench
    mix = bench.pass_mix_ceiling(iters=500, reps=2)
    assert 0 < mix["pass_mix"] <= mix["mfma_sustained"] * 1.02
    assert mix["mfma_sustained"] <= PEAK_BF16_TFLOPS * 1.02


def test_l2_ceilings_exceed_hbm_and_order():
    import bench
    l2, _ = bench.l2_read_ceiling(regions_mb=(2,), pass_bytes=2e9, reps=2)
    lds, _ = bench.l2_read_ceiling(regions_mb=(2,), mode=2, grid=2560, pass_bytes=2e9, reps=2)
    assert l2 > PEAK_HBM_GBS and lds > PEAK_HBM_GBS
    assert lds <= l2 * 1.05
