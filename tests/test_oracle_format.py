"""Pins of the CPU oracle's format arithmetic against the pages, closed forms, exact
rationals and library routines (no GPU)."""
import json
import math
import os
from fractions import Fraction as Fr

import numpy as np
import pytest
import torch

from oracle import exact

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- E2M1 element format

def test_e2m1_values_match_page_list(orc):
    g = gold("e2m1_values.json")
    vals = sorted({orc.e2m1_value(c) for c in range(16)})
    mags = sorted({abs(v) for v in vals})
    assert mags == g["magnitudes"]
    assert max(vals) == g["max"] and min(vals) == -g["max"]
    # 16 codes: +-0 decode to the same zero, so 15 distinct values
    assert len(vals) == 15 and len(range(16)) == g["n_codes"]


def test_e2m1_decode_is_bias1_sign_exp_mantissa(orc):
    # closed form for a 1-2-1 float with exponent bias 1 and a subnormal at exponent 0
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        mag = m * 0.5 if e == 0 else (1 + m / 2) * 2.0 ** (e - 1)
        assert orc.e2m1_value(c) == (-mag if s else mag)


# ---------------------------------------------------------------- E4M3 scale format

def test_e4m3_has_126_positive_candidates(orc):
    g = gold("e4m3_candidates.json")
    vals = [orc.e4m3_value(b) for b in range(128)]
    pos = [v for v in vals if v == v and v > 0]
    assert len(pos) == g["n_positive_nonzero"] == 126
    assert all(a < b for a, b in zip(pos, pos[1:])), "candidate order must be increasing"
    assert max(pos) == 448.0 and min(pos) == 2.0 ** -9
    assert math.isnan(vals[0x7F]) and vals[0] == 0.0


def test_e4m3_decode_matches_torch_float8_e4m3fn(orc):
    b = torch.arange(128, dtype=torch.int32).to(torch.uint8)
    ref = b.view(torch.float8_e4m3fn).double().numpy()
    for i in range(128):
        v = orc.e4m3_value(i)
        if math.isnan(ref[i]):
            assert math.isnan(v)
        else:
            assert v == ref[i], i


def test_e4m3_decode_matches_exact(orc):
    for b in range(127):
        assert Fr(orc.e4m3_value(b)) == exact.e4m3(b)


# ---------------------------------------------------------------- bf16 rounding

def test_bf16_rne_matches_torch(orc):
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(3000).astype(np.float32) * np.float32(10.0) ** rng.integers(-30, 30, 3000).astype(np.float32),
        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.0e38, 1e-40, -1e-40,
                  np.float32(1.0) + np.float32(2.0 ** -8), np.float32(1.0) + np.float32(3 * 2.0 ** -9)],
                 dtype=np.float32)])
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = orc.bf16_rne_array(x)
    assert np.array_equal(got, ref)


# ---------------------------------------------------------------- tensor scale

def test_tensor_scale_is_fp32_division(orc):
    rng = np.random.default_rng(2)
    for _ in range(200):
        x = (rng.standard_normal(64) * 10.0 ** rng.uniform(-6, 6)).astype(np.float32)
        amax = np.max(np.abs(x))
        assert orc.tensor_scale(x) == np.float32(amax) / np.float32(2688.0)
    assert orc.tensor_scale(np.zeros(32, np.float32)) == 1.0
    # a tensor whose max maps exactly onto the top E4M3 value: 84 / 2688 = 2^-5
    assert orc.tensor_scale(np.array([84.0, -3.0], np.float32)) == np.float32(2.0 ** -5)


# ---------------------------------------------------------------- max-scaling byte

def test_max_byte_matches_exact_rationals(orc):
    rng = np.random.default_rng(3)
    for _ in range(3000):
        amax = np.float32(abs(rng.standard_normal()) * 10.0 ** rng.uniform(-4, 3))
        S = np.float32(10.0 ** rng.uniform(-6, 1))
        assert orc.max_byte(amax, S) == exact.max_byte(Fr(float(amax)), Fr(float(S)))


@pytest.mark.parametrize("S", [1.0, 0.75, 2.0 ** -7])
def test_max_byte_ties_go_to_even_byte(orc, S):
    # amax exactly on the midpoint between consecutive E4M3 values (x 6S): exact in fp32
    for b in range(0, 126):
        mid = (Fr(orc.e4m3_value(b)) + Fr(orc.e4m3_value(b + 1))) / 2
        amax = mid * 6 * Fr(S)
        if Fr(float(np.float32(float(amax)))) != amax:
            continue
        got = orc.max_byte(float(amax), S)
        want = b if b % 2 == 0 else b + 1
        assert got == max(want, 1), (b, got)


def test_max_byte_saturates_and_floors(orc):
    assert orc.max_byte(1e30, 1.0) == 0x7E            # far above 448 * 6
    assert orc.max_byte(448.0 * 6, 1.0) == 0x7E
    assert orc.max_byte(1e-30, 1.0) == 0x01           # rounds to 0 -> smallest candidate
    assert orc.max_byte(0.0, 1.0) == 0x00             # all-zero block


def test_max_byte_matches_torch_cast_away_from_ties(orc):
    rng = np.random.default_rng(4)
    for _ in range(2000):
        amax = np.float32(abs(rng.standard_normal()) * 10.0 ** rng.uniform(-2, 2.5))
        S = np.float32(1.0)
        q = float(amax) / 6.0
        if q >= 448.0 or q < 2.0 ** -9:
            continue
        ref = torch.tensor([q], dtype=torch.float64).to(torch.float8_e4m3fn).view(torch.uint8).item()
        assert orc.max_byte(amax, S) == ref


# ---------------------------------------------------------------- element code

def test_code_tie_table_at_unit_scale(orc):
    # S = 1 and byte 0x38 (= 1.0), so |x|/(sS) = |x|: ties go to the even grid index
    table = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0,
             6.5: 6.0, 100.0: 6.0, 0.2: 0.0, 0.3: 0.5, 5.01: 6.0}
    assert orc.e4m3_value(0x38) == 1.0
    for x, v in table.items():
        for sgn in (1, -1):
            c = orc.e2m1_code(sgn * x, 0x38, 1.0)
            assert orc.e2m1_value(c) == (sgn * v if v else 0.0), (x, c)
            if v == 0.0:
                assert c == 0, "zero magnitude never carries the sign bit"


def test_code_matches_library_round_half_even(orc):
    # on [0,2) the grid is multiples of 0.5, on [2,4) of 1, on [4,6] of 2: numpy's
    # round-half-even to those spacings is the E2M1 round-to-nearest-even
    y = np.arange(0, 6.5, 1 / 64, dtype=np.float32)
    for v in y:
        if v < 2:
            r = np.round(2 * v) / 2
        elif v < 4:
            r = np.round(v)
        else:
            r = 2 * np.round(v / 2)
        r = min(r, 6.0)
        assert orc.e2m1_value(orc.e2m1_code(v, 0x38, 1.0)) == r, v


def test_code_matches_exact_rationals(orc):
    rng = np.random.default_rng(5)
    for _ in range(4000):
        S = np.float32(10.0 ** rng.uniform(-5, 0))
        byte = int(rng.integers(1, 127))
        sS = orc.e4m3_value(byte) * float(S)
        x = np.float32(rng.uniform(-7, 7) * sS)
        assert orc.e2m1_code(x, byte, S) == exact.code(Fr(float(x)), byte, Fr(float(S)))


def test_code_at_exact_midpoints_with_general_scale(orc):
    # S with a full 24-bit mantissa: midpoints M*s*S are exact doubles but not floats;
    # take the two floats around each midpoint and check against exact rationals
    rng = np.random.default_rng(6)
    for _ in range(300):
        S = np.float32(rng.uniform(0.5, 1.0) * 2.0 ** -5)
        byte = int(rng.integers(1, 127))
        for M in (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0):
            t = M * orc.e4m3_value(byte) * float(S)
            lo = np.float32(t)
            for x in (np.nextafter(lo, np.float32(0)), lo, np.nextafter(lo, np.float32(np.inf))):
                assert orc.e2m1_code(x, byte, S) == exact.code(Fr(float(x)), byte, Fr(float(S)))


# ---------------------------------------------------------------- dequantisation

def test_dequant_is_one_rounding_of_exact_product(orc):
    rng = np.random.default_rng(7)
    for _ in range(3000):
        S = np.float32(10.0 ** rng.uniform(-8, 2))
        byte = int(rng.integers(1, 127))
        code = int(rng.integers(0, 16))
        ex = exact.dequant_exact(code, byte, Fr(float(S)))
        want = np.float32(float(ex))  # ex has <= 30 bits, so float(ex) is exact
        got = orc.dequant_value(code, byte, S)
        assert got == want or (want == 0 and got == 0)
    assert np.signbit(orc.dequant_value(8, 0x38, 1.0)) == False  # noqa: E712


# ---------------------------------------------------------------- the worked example

def test_worked_example_unit_tensor_scale(orc):
    g = gold("worked_example.json")
    x = np.array(g["block"], np.float32)
    b = orc.max_byte(np.max(np.abs(x)), 1.0)
    assert orc.e4m3_value(b) == g["scale"] == 84 / 6
    mags = sorted({abs(orc.e2m1_value(k)) * g["scale"] for k in range(8)})
    assert mags == g["magnitudes"]
    dq, codes, sc = orc.fakequant(x.reshape(1, 16), 1.0)
    assert set(np.abs(dq).ravel().tolist()) <= set(g["magnitudes"])
    assert dq[0, 0] == 84.0
    small = np.abs(x) < g["zero_below"]
    assert np.all(dq[0, small] == 0.0)


def test_worked_example_automatic_tensor_scale(orc):
    g = gold("worked_example.json")
    x = np.array(g["block"], np.float32).reshape(1, 16)
    S = orc.tensor_scale(x)
    assert S == np.float32(2.0 ** -5)
    b = orc.max_byte(84.0, S)
    assert b == 0x7E and orc.e4m3_value(b) * float(S) == 14.0
    dq_auto, _, _ = orc.fakequant(x, S)
    dq_unit, _, _ = orc.fakequant(x, 1.0)
    assert np.array_equal(dq_auto, dq_unit)


# ---------------------------------------------------------------- invariants

def _rand_tensor(seed, rows=32, cols=256):
    rng = np.random.default_rng(seed)
    x = rng.standard_t(3, size=(rows, cols)).astype(np.float32)
    x[:, 5] *= 30
    return x


def test_every_output_on_scaled_grid(orc):
    x = _rand_tensor(8)
    S = orc.tensor_scale(x)
    dq, codes, sc = orc.fakequant(x, S)
    for r in range(x.shape[0]):
        for b in range(x.shape[1] // 16):
            s = orc.e4m3_value(sc[r, b])
            grid = {np.float32(float(exact.GRID[k] * Fr(s) * Fr(float(S)))) for k in range(8)}
            blk = dq[r, b * 16:(b + 1) * 16]
            assert set(np.abs(blk).tolist()) <= {float(g) for g in grid}
            assert np.all(np.abs(blk) <= np.float32(6.0 * s * float(S)))


def test_fakequant_is_idempotent_with_fixed_scale(orc):
    x = _rand_tensor(9)
    S = orc.tensor_scale(x)
    dq1, c1, s1 = orc.fakequant(x, S)
    assert np.all(s1 >= 8), "all block scales normal (the precondition of this invariant)"
    dq2, c2, s2 = orc.fakequant(dq1, S)
    assert np.array_equal(dq1, dq2)
    assert np.array_equal(s1, s2) and np.array_equal(c1, c2)
    # with the bytes held fixed it holds for any bytes
    dq3, _, _ = orc.fakequant(dq1, S, s1)
    assert np.array_equal(dq1, dq3)


def test_packing_order_low_nibble_first(orc):
    x = np.array([[1.0, -2.0] + [0.0] * 14], np.float32)
    sc = np.array([[0x38]], np.uint8)
    codes = orc.quantize(x, 1.0, sc)
    # 1.0 is grid index 2, -2.0 is sign | index 4
    assert codes[0, 0] == (2 | ((8 | 4) << 4))
    assert np.all(codes[0, 1:] == 0)
    y = orc.dequantize(codes, sc, 1.0, 1, 16)
    assert y[0, 0] == 1.0 and y[0, 1] == -2.0


def test_zero_block_gets_zero_byte_and_positive_zero(orc):
    x = np.zeros((2, 32), np.float32)
    x[1, 16:] = -0.0
    dq, codes, sc = orc.fakequant(x, 1.0)
    assert np.all(sc == 0) and np.all(codes == 0)
    assert not np.any(np.signbit(dq))


def test_given_byte_reads_the_e4m3_magnitude(orc):
    """A given block byte acts as its E4M3FN magnitude: torch's float8_e4m3fn decode of
    b | 0x80 is the negative of b's value, and the oracle codes and dequantises with |value|;
    0x7F and 0xFF decode to NaN there and, like 0x00 and 0x80 (zero), code a block as zeros."""
    import torch
    rng = np.random.default_rng(3)
    S = np.float32(0.01)
    dec = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    for b in range(1, 0x7F):
        assert dec[b | 0x80] == -dec[b] == -orc.e4m3_value(b)
        x = (rng.uniform(-7, 7, 16) * dec[b] * S).astype(np.float32)
        for v in x:
            c = orc.e2m1_code(float(v), b, S)
            assert orc.e2m1_code(float(v), b | 0x80, S) == c
            assert orc.dequant_value(c, b | 0x80, S) == orc.dequant_value(c, b, S)
    assert np.isnan(dec[0x7F]) and np.isnan(dec[0xFF]) and dec[0x80] == 0
    for b in (0x00, 0x7F, 0x80, 0xFF):
        for v in (0.0, 1e-3, -2.0, 5.0):
            assert orc.e2m1_code(v, b, S) == 0
            assert orc.dequant_value(0x7, b, S) == 0.0
