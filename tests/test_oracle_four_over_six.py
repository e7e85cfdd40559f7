"""Pins of the oracle's Four Over Six selector: its two candidate bytes against exact
rationals, its choice against exact objectives, closed-form blocks where the answer is
known, the tie rule, and the ordering MSE <= Four Over Six <= max (no GPU)."""
from fractions import Fraction as Fr

import numpy as np
import pytest

from oracle import exact
from scale_search_weights_amd import synth


def _fp32_round(q: Fr) -> Fr:
    return Fr(float(np.float32(float(q))))  # q has <= 30 significant bits: float(q) exact


@pytest.fixture(scope="module")
def tiny():
    w, _ = synth.tiny(0)
    return w.numpy()


@pytest.mark.parametrize("k", [4, 6])
def test_divisor_bytes_match_exact(orc, k):
    rng = np.random.default_rng(k)
    S = np.float32(0.0371)
    for a in np.abs(rng.standard_normal(400) * 40).astype(np.float32):
        assert orc.byte_for_divisor(float(a), float(S), k) == \
            exact.byte_for_divisor(Fr(float(a)), Fr(float(S)), k), (a, k)
    # amax / (k S) exactly on the midpoint between two E4M3 values (S = 1/4): ties go to
    # the even byte
    for b in (3, 17, 64, 90, 125):
        mid = (exact.e4m3(b) + exact.e4m3(b + 1)) / 2 * k * Fr(1, 4)
        got = orc.byte_for_divisor(float(mid), 0.25, k)
        assert got == exact.byte_for_divisor(mid, Fr(1, 4), k) == (b if b % 2 == 0 else b + 1)


def test_choice_matches_exact_objectives(orc, tiny):
    """Candidates equal the exact bytes; the choice is the exact argmin of the two
    objectives (dq rounded to fp32 as stored) unless they are within 1e-5 of each other."""
    w = tiny
    S = orc.tensor_scale(w)
    got, obj = orc.scales_four_over_six(w, S, with_obj=True)
    Sx = Fr(float(S))
    close = 0
    for r in range(0, w.shape[0], 3):
        for b in range(w.shape[1] // 16):
            xs = [Fr(float(v)) for v in w[r, b * 16:(b + 1) * 16]]
            amax = max(abs(x) for x in xs)
            c6, c4 = exact.byte_for_divisor(amax, Sx, 6), exact.byte_for_divisor(amax, Sx, 4)
            e6 = exact.block_sq_error_exact(xs, c6, Sx, _fp32_round)
            e4 = exact.block_sq_error_exact(xs, c4, Sx, _fp32_round)
            assert got[r, b] in (c6, c4)
            lo, hi = min(e6, e4), max(e6, e4)
            if hi - lo <= lo * Fr(1, 10 ** 5):
                close += 1
            else:
                assert got[r, b] == (c4 if e4 < e6 else c6), (r, b)
    assert close < 10


def test_block_on_the_four_grid_takes_the_second_candidate(orc):
    """Values u * {4, 3, 2, 1.5, 1, 0.5, 0} with u an E4M3 value (S = 1): amax / 4 = u, so
    the second candidate reproduces the block exactly, while amax / 6 does not."""
    u = float(exact.e4m3(0x40))  # 2.0
    vals = np.array([4, -3, 2, 1.5, -1, 0.5, 0, 3, -4, 2, 1, -0.5, 1.5, 0, 4, -2],
                    dtype=np.float32) * u
    w = vals.reshape(1, 16)
    got, obj = orc.scales_four_over_six(w, 1.0, with_obj=True)
    assert got[0, 0] == 0x40 and obj[0, 0] == 0.0
    c6 = orc.max_byte(float(np.abs(vals).max()), 1.0)
    assert c6 != 0x40 and orc.block_sq_error(vals, c6, 1.0) > 0.0


def test_equal_objectives_take_the_smaller_byte(orc):
    """A lone value 24 * 2^j maps exactly onto 6 * E4M3 and onto 4 * E4M3: both candidates
    have objective 0, and the smaller byte (the max-scaling one) wins."""
    for j in (-3, 0, 2):
        v = np.float32(24.0 * 2.0 ** j)
        w = np.zeros((1, 16), dtype=np.float32)
        w[0, 5] = v
        got, obj = orc.scales_four_over_six(w, 1.0, with_obj=True)
        c6, c4 = orc.byte_for_divisor(float(v), 1.0, 6), orc.byte_for_divisor(float(v), 1.0, 4)
        assert c4 > c6 and exact.e4m3(c6) == Fr(4) * Fr(2) ** j
        assert got[0, 0] == c6 and obj[0, 0] == 0.0


def test_between_mse_and_max(orc, tiny):
    w = tiny
    S = orc.tensor_scale(w)
    _, o46 = orc.scales_four_over_six(w, S, with_obj=True)
    _, omse = orc.scales_mse(w, S, with_obj=True)
    mx = orc.scales_max(w, S)
    for r in range(w.shape[0]):
        for b in range(w.shape[1] // 16):
            e_max = orc.block_sq_error(w[r, b * 16:(b + 1) * 16], mx[r, b], S)
            assert omse[r, b] <= o46[r, b] <= e_max


def test_worked_example_block(orc):
    """[BT] "Why blocks" block (84 among values near 1-2), S = 1: the candidates are 14
    (0x56) and 21 -> 20 (0x5A, the even neighbour on the tie); 14 keeps the smaller error."""
    import json, os
    ex = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")))
    vals = np.array(ex["block"], dtype=np.float32).reshape(1, 16)
    assert orc.byte_for_divisor(84.0, 1.0, 6) == 0x56
    assert orc.byte_for_divisor(84.0, 1.0, 4) == 0x5A
    got, obj = orc.scales_four_over_six(vals, 1.0, with_obj=True)
    assert got[0, 0] == 0x56
    assert obj[0, 0] == orc.block_sq_error(vals[0], 0x56, 1.0)
