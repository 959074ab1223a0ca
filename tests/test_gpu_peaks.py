"""Calibration kernels (libmla_peaks.so) on the GPU: every figure the bench
reports as a measured peak is produced and lies between a tenth of and the
vendor's peak (HBM 8 TB/s, dense matrix ops 2.5 / 5.0 PFLOP/s)."""
import pytest
import torch

import bench

pytestmark = pytest.mark.gpu


def test_measured_peaks_are_plausible():
    res = bench.measure_peaks(torch, "cuda:0", reps=3, patterns=("tiles", "rows1152", "rows576"))
    for key in ("stream_lds_grid256_inflight2_nt", "read_grid4096", "pattern_tiles_GBps",
                "pattern_rows1152_GBps", "pattern_rows576_GBps"):
        assert 800.0 < res[key] < bench.PEAK_HBM_GBPS, (key, res[key])
    assert 250.0 < res["mfma_bf16_TFLOPs"] < bench.PEAK_MFMA_TFLOPS["bf16"]
    assert 500.0 < res["mfma_fp8_TFLOPs"] < bench.PEAK_MFMA_TFLOPS["fp8"]
