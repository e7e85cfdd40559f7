"""Row-by-row check of GPTQ codes from the GPU against the oracle (used by the GPTQ GPU
tests; not a test module itself).

A code is decided on a double-precision value whose last bits depend on the order of the
sums that made it, so at a value within a hair of a rounding midpoint both roundings are
correct, and after such a column the rest of the row follows from whichever was taken.
The check therefore walks each row that differs: at its first differing column the
oracle's value must lie within tie_tol * s * S of a midpoint; the oracle then takes the
other rounding there too (its `flips` option: the grid neighbour across that midpoint) and
recomputes the row, and the walk continues from there. Every column of every row is thus
either identical to the oracle's or a verified near-tie, and every expected code is the
oracle's own.
"""
import numpy as np

MIDS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])


def unpack(codes: np.ndarray) -> np.ndarray:
    return np.stack([codes & 15, codes >> 4], axis=-1).reshape(codes.shape[0], -1)


def check_rows(got, w, S, scales, U, orc, tie_tol, max_flips=64):
    """got: packed GPU codes [rows, cols/2]; w (fp32), scales and U as the oracle takes
    them. Returns the number of near-ties the rows went through."""
    g = unpack(np.asarray(got))
    w = np.ascontiguousarray(w, dtype=np.float32)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    pending = np.flatnonzero((g != unpack(orc.gptq(w, S, scales, U=U))).any(axis=1))
    flips: dict[int, list[int]] = {}
    ties = 0
    while pending.size:
        F = np.full((pending.size, max_flips), -1, np.int64)
        for i, r in enumerate(pending):
            fr = flips.get(int(r), [])
            F[i, :len(fr)] = fr
        c, v = orc.gptq(w[pending], S, scales[pending], U=U, return_v=True, flips=F)
        c = unpack(c)
        nxt = []
        for i, r in enumerate(pending):
            r = int(r)
            d = np.flatnonzero(g[r] != c[i])
            if d.size == 0:
                continue
            j = int(d[0])
            prev = flips.get(r, [])
            assert not prev or j > prev[-1], f"row {r}: the other rounding at column {prev[-1]} differs too"
            sS = orc.e4m3_value(int(scales[r, j // 16])) * float(S)
            dist = float(np.min(np.abs(abs(v[i, j]) - MIDS * sS)) / sS)
            assert dist <= tie_tol, (f"row {r} col {j}: codes {g[r, j]} vs {c[i, j]}, "
                                     f"{dist:.3g} s S from a midpoint")
            flips.setdefault(r, []).append(j)
            assert len(flips[r]) < max_flips, f"row {r}: more than {max_flips} near-ties"
            ties += 1
            nxt.append(r)
        pending = np.array(nxt, dtype=np.int64)
    return ties
