"""Exact-rational NVFP4 micro-oracle (fractions.Fraction), for pinning the C oracle.

TEST INFRASTRUCTURE ONLY. Slow by design: it is meant for single blocks and tiny tensors.

It restates the format from the pages with no floating point at all:
* E2M1 magnitudes 0, 1/2, 1, 3/2, 2, 3, 4, 6 ([BT] "Why do we need a scale");
* E4M3FN values m/512 (exponent field 0) or (1 + m/8) 2^(e-7) ([LH] counts 126 positive
  non-zero ones);
* nearest-value rounding with ties to the even index ([QAD] sec. 2.1; the tie rule is a
  reading);
and evaluates objectives exactly, so argmins here are those of the real-valued objective.
"""
from __future__ import annotations

from fractions import Fraction as Fr

GRID = [Fr(0), Fr(1, 2), Fr(1), Fr(3, 2), Fr(2), Fr(3), Fr(4), Fr(6)]


def e4m3(byte: int) -> Fr:
    e, m = (byte >> 3) & 15, byte & 7
    if e == 0:
        return Fr(m, 512)
    return Fr(8 + m, 8) * Fr(2) ** (e - 7)


def nearest_index(values, y: Fr) -> int:
    """Index of the value nearest to y; on a tie the even index (values ascending)."""
    best_k, best_d = None, None
    for k, v in enumerate(values):
        d = abs(y - v)
        if best_d is None or d < best_d or (d == best_d and k % 2 == 0):
            best_k, best_d = k, d
    return best_k


E4M3_VALUES = [e4m3(b) for b in range(127)]  # bytes 0x00..0x7E


def max_byte(amax: Fr, S: Fr) -> int:
    """E4M3 byte nearest to amax / (6 S), saturating at 448 and at least 1 if amax > 0."""
    return byte_for_divisor(amax, S, 6)


def byte_for_divisor(amax: Fr, S: Fr, k: int) -> int:
    """E4M3 byte nearest to amax / (k S) (ties to the even byte), saturating at 448 and at
    least 1 if amax > 0."""
    if amax == 0:
        return 0
    q = Fr(amax) / (k * Fr(S))
    if q >= 448:
        return 126
    b = nearest_index(E4M3_VALUES, q)
    return max(b, 1)


def code(x: Fr, byte: int, S: Fr) -> int:
    if byte == 0:
        return 0
    y = abs(Fr(x)) / (e4m3(byte) * Fr(S))
    k = 7 if y >= 6 else nearest_index(GRID, y)
    return (8 | k) if (x < 0 and k > 0) else k


def dequant_exact(c: int, byte: int, S: Fr) -> Fr:
    """Exact (unrounded) dequantised value G_k * s * S with the code's sign."""
    v = GRID[c & 7] * e4m3(byte) * Fr(S) if byte else Fr(0)
    return -v if (c & 8) else v


def block_sq_error_exact(xs, byte: int, S: Fr, dq_round=None) -> Fr:
    """Sum of (dq_i - x_i)^2 in exact arithmetic. ``dq_round`` maps the exact dequantised
    value to the stored one (e.g. rounding to fp32); identity if None."""
    tot = Fr(0)
    for x in xs:
        x = Fr(x)
        dq = dequant_exact(code(x, byte, S), byte, S)
        if dq_round is not None:
            dq = dq_round(dq)
        tot += (dq - x) ** 2
    return tot


def mse_ranking(xs, S: Fr, dq_round=None):
    """All 126 (exact objective, byte) pairs, ascending."""
    return sorted((block_sq_error_exact(xs, b, S, dq_round), b) for b in range(1, 127))


def quad_form(d, H) -> Fr:
    return sum(Fr(d[i]) * Fr(H[i][j]) * Fr(d[j]) for i in range(len(d)) for j in range(len(d)))
