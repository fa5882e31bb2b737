"""Checks of the seeded input generators (shapes, distributions, determinism)."""

import numpy as np
import torch

from workloads import (
    QK_WORKLOADS,
    RMS_WORKLOADS,
    f32_to_bf16_bits,
    make_rms_inputs,
    outlier_rows,
)


def test_f32_to_bf16_matches_torch():
    rng = np.random.default_rng(5)
    f = (rng.standard_normal(200_000) * 10.0 ** rng.integers(-30, 30, 200_000)).astype(np.float32)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f32_to_bf16_bits(f), ref)


def test_algorithmic_bytes():
    assert RMS_WORKLOADS["rms_16384x16384"].algorithmic_bytes == 1_073_774_592
    assert RMS_WORKLOADS["rms_1024x4096"].algorithmic_bytes == 16_785_408
    assert RMS_WORKLOADS["rms_8192x8192"].algorithmic_bytes == 268_451_840
    assert RMS_WORKLOADS["rms_4096x32768"].algorithmic_bytes == 536_936_448
    assert QK_WORKLOADS["qk_256"].algorithmic_bytes == 5_245_440


def test_small_workload_distribution_and_determinism():
    wl = RMS_WORKLOADS["rms_1024x4096"]
    x, w, eps = make_rms_inputs(wl)
    x2, w2, _ = make_rms_inputs(wl)
    assert np.array_equal(x, x2) and np.array_equal(w, w2)
    assert x.shape == (1024, 4096) and w.shape == (4096,) and eps == 1e-6
    xv = (x.astype(np.uint32) << 16).view(np.float32)
    wv = (w.astype(np.uint32) << 16).view(np.float32)
    assert abs(xv.mean()) < 0.01 and abs(xv.std() - 1) < 0.01
    assert wv.min() >= 0.5 and wv.max() <= 1.5 and abs(wv.mean() - 1.0) < 0.02
    xr, _, _ = make_rms_inputs(wl, rows=10)
    assert np.array_equal(xr, x[:10])


def test_outlier_rows_recipe():
    wl = RMS_WORKLOADS["rms_8192x8192"]
    idx = outlier_rows(wl)
    assert len(idx) == 81 and len(np.unique(idx)) == 81
