"""Pins of the oracle's straight-through backward (gradient clamp) and moving-average
scale: closed forms, identities and exact arithmetic (no GPU)."""
from fractions import Fraction as Fr

import numpy as np


def test_clamp_identity_without_bound(orc):
    g = (np.random.default_rng(0).standard_normal(4000) * 100).astype(np.float32)
    assert np.array_equal(orc.ste_backward(g, np.inf), g)


def test_clamp_matches_numpy_clip_and_is_odd(orc):
    g = (np.random.default_rng(1).standard_normal(4000) * 3).astype(np.float32)
    for c in (0.5, 1.0, 2.75):
        out = orc.ste_backward(g, c)
        assert np.array_equal(out, np.clip(g, -np.float32(c), np.float32(c)))
        assert np.array_equal(orc.ste_backward(-g, c), -out)


def test_clamp_edge_values(orc):
    g = np.array([1.0, -1.0, 0.0, -0.0, 1e-45, 3.0e38], np.float32)
    out = orc.ste_backward(g, 1.0)
    want = np.array([1.0, -1.0, 0.0, -0.0, 1e-45, 1.0], np.float32)
    assert np.array_equal(out.view(np.uint32), want.view(np.uint32))  # -0 and denormals kept


def _rn32(q: Fr) -> np.float32:
    """q rounded once to the nearest fp32 (ties to even), from exact comparisons."""
    f = np.float32(float(q))
    best = None
    for c in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        d = abs(Fr(float(c)) - q)
        key = (d, int(np.array([c], np.float32).view(np.uint32)[0]) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def test_ema_exact_arithmetic(orc):
    """S = fmaf(m, S_prev, fp32(fp32(1 - m) * S_batch)): checked with exact rationals and a
    single final rounding of the fma."""
    rng = np.random.default_rng(2)
    prev = rng.uniform(1e-4, 1e-1, 200).astype(np.float32)
    batch = rng.uniform(1e-4, 1e-1, 200).astype(np.float32)
    for m in (0.9, 0.99, 0.5):
        got = orc.scale_ema(prev, batch, m)
        mf = np.float32(m)
        a = np.float32(np.float32(1.0) - mf)
        for p, b, g in zip(prev, batch, got):
            bb = np.float32(a * b)  # fp32 product, rounded
            exact = Fr(float(mf)) * Fr(float(p)) + Fr(float(bb))
            assert g == _rn32(exact)


def test_ema_fixed_point_and_extremes(orc):
    S = np.array([0.125, 3.0, 1e-30], np.float32)
    # a constant batch scale is a fixed point when the arithmetic is exact
    assert np.array_equal(orc.scale_ema(S, S, 0.5), S)
    assert np.array_equal(orc.scale_ema(S, S * 4, 0.0), S * 4)   # momentum 0: the new value
    assert np.array_equal(orc.scale_ema(S, S * 4, 1.0), S)       # momentum 1: frozen


def test_clamp_passes_nan_and_clamps_infinities(orc):
    g = np.array([np.nan, np.inf, -np.inf], np.float32)
    out = orc.ste_backward(g, 2.0)
    assert np.isnan(out[0]) and out[1] == 2.0 and out[2] == -2.0
