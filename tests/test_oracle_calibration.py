"""Pins of the oracle's static activation calibration (histogram of |x| with one bin per
bf16 magnitude, clip value from a fraction of the calibration values) against order
statistics from a sort, the max calibration, and closed-form cases (no GPU)."""
import math

import numpy as np
import pytest

from scale_search_weights_amd import synth


def _bf16_data(seed, n=200_000):
    x = synth.activation(seed, tokens=n // 512, hidden=512).float().numpy().ravel()
    return x  # bf16 values, widened exactly


def _expected_S(clip: np.float32) -> np.float32:
    if clip == 0:
        return np.float32(1.0)
    S = np.float32(clip) / np.float32(2688.0)  # IEEE fp32 division
    return max(S, np.float32(np.finfo(np.float32).tiny))


@pytest.mark.parametrize("frac", [0.5, 0.9, 0.99, 0.999, 0.9999, 1.0])
def test_bf16_clip_is_the_order_statistic(orc, frac):
    x = _bf16_data(1)
    h = orc.calib_histogram(x)
    assert int(h.sum()) == x.size
    k = max(1, math.ceil(frac * x.size))
    v = np.sort(np.abs(x))[k - 1]
    assert orc.calib_scale(h, frac) == _expected_S(v)


@pytest.mark.parametrize("frac", [0.9, 0.9999])
def test_fp32_clip_is_the_order_statistic_truncated_to_bf16(orc, frac):
    x = (np.random.default_rng(3).standard_normal(100_000) * 3).astype(np.float32)
    h = orc.calib_histogram(x)
    k = math.ceil(frac * x.size)
    v = np.sort(np.abs(x))[k - 1]
    vt = (np.array([v], np.float32).view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)[0]
    assert vt <= v and orc.calib_scale(h, frac) == _expected_S(vt)


def test_fraction_one_is_the_max_calibration(orc):
    x = _bf16_data(2)
    assert orc.calib_scale(orc.calib_histogram(x), 1.0) == orc.tensor_scale(x)


def test_streaming_batches_equal_one_batch(orc):
    a, b, c = _bf16_data(4, 30_000), _bf16_data(5, 50_000), _bf16_data(6, 20_000)
    h = orc.calib_histogram(a)
    orc.calib_histogram(b, h)
    orc.calib_histogram(c, h)
    assert np.array_equal(h, orc.calib_histogram(np.concatenate([a, b, c])))


def test_a_lone_outlier_is_clipped(orc):
    x = np.full(1000, 0.5, np.float32)
    x[123] = -1000.0
    h = orc.calib_histogram(x)
    assert orc.calib_scale(h, 0.999) == _expected_S(np.float32(0.5))
    assert orc.calib_scale(h, 1.0) == _expected_S(np.float32(1000.0))


def test_zero_denormal_and_signed_zero(orc):
    z = np.array([0.0, -0.0, 0.0, -0.0], np.float32)
    h = orc.calib_histogram(z)
    assert h[0] == 4 and orc.calib_scale(h, 1.0) == np.float32(1.0)
    d = np.array([1e-40, -3e-41, 0.0], np.float32)
    h = orc.calib_histogram(d)
    assert orc.calib_scale(h, 1.0) == np.finfo(np.float32).tiny
