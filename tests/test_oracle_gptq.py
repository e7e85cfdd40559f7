"""Pins of the oracle's full Gram matrix and GPTQ rounding (no GPU): integer closed forms,
the independent conditional-minimiser (optimal brain surgeon) formulation of GPTQ's update
solved directly, special cases that reduce to plain rounding, and exact invariances."""
import numpy as np
import pytest


def _problem(seed, rows=6, cols=48, tokens=200, corr=0.8):
    rng = np.random.default_rng(seed)
    base = rng.standard_normal((tokens, 1))
    X = (corr * base + rng.standard_normal((tokens, cols))).astype(np.float32)  # correlated
    w = (rng.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    return w, X


def test_full_hessian_integer_closed_form(orc):
    rng = np.random.default_rng(0)
    X = rng.integers(-3, 4, (50, 32)).astype(np.float32)
    H = orc.full_hessian(X)
    Xi = X.astype(np.int64)
    assert np.array_equal(H, (Xi.T @ Xi).astype(np.float64))


def test_full_hessian_library_matmul_agrees(orc):
    _, X = _problem(12, cols=96, tokens=700)
    H, Hb = orc.full_hessian(X), orc.full_hessian_blas(X)
    assert np.abs(H - Hb).max() <= 1e-13 * np.abs(H).max()


def test_full_hessian_diagonal_blocks_match_block_hessian(orc):
    _, X = _problem(1, cols=64, tokens=300)
    H = orc.full_hessian(X)
    Hb = orc.block_hessian(X)
    for b in range(4):
        assert np.allclose(H[16 * b:16 * b + 16, 16 * b:16 * b + 16], Hb[b], rtol=1e-12, atol=0)
    assert np.array_equal(H, H.T)


def test_code_d_agrees_with_fp32_rule_and_is_exact(orc):
    rng = np.random.default_rng(2)
    S = np.float32(1.7e-3)
    for byte in (1, 17, 56, 90, 126):
        for x in (rng.standard_normal(200) * orc.e4m3_value(byte) * float(S) * 3).astype(np.float32):
            assert orc.e2m1_code_d(float(x), byte, S) == orc.e2m1_code(x, byte, S)
    # a double one ulp above the midpoint 2.5 s S rounds up; exactly on it ties to even (2.0)
    byte = 56
    mid = 2.5 * orc.e4m3_value(byte) * float(S)
    assert orc.e2m1_code_d(mid, byte, S) == 4            # k = 4 -> 2.0 (even index)
    assert orc.e2m1_code_d(np.nextafter(mid, 1.0), byte, S) == 5
    assert orc.e2m1_code_d(-np.nextafter(mid, 1.0), byte, S) == 8 | 5
    assert orc.e2m1_code_d(-0.0, byte, S) == 0


def test_factor_is_inverse_cholesky(orc):
    _, X = _problem(3, cols=40)
    H = orc.full_hessian(X)
    U = orc.gptq_factor(H, 0.01)
    lam = 0.01 * np.trace(H) / 40
    Hd = H + lam * np.eye(40)
    assert np.allclose(np.tril(U, -1), 0) and (np.diag(U) > 0).all()
    assert np.allclose(U.T @ U @ Hd, np.eye(40), atol=1e-10)


def test_factor_two_by_two_closed_form(orc):
    H = np.array([[4.0, 1.5], [1.5, 2.0]])
    U = orc.gptq_factor(H, 0.0)
    det = 4.0 * 2.0 - 1.5 * 1.5
    hi11, hi12, hi22 = 2.0 / det, -1.5 / det, 4.0 / det
    u11 = np.sqrt(hi11)
    u12 = hi12 / u11
    assert np.allclose(U, [[u11, u12], [0.0, np.sqrt(hi22 - u12 * u12)]], rtol=1e-14)


def _rtn(orc, w, S, sc):
    return orc.quantize(w, S, sc)


def test_diagonal_or_zero_hessian_is_plain_rounding(orc):
    w, _ = _problem(4, rows=8, cols=64)
    S = orc.tensor_scale(w)
    sc = orc.scales_max(w, S)
    rng = np.random.default_rng(4)
    for H in (np.diag(rng.uniform(0.5, 3.0, 64)), np.zeros((64, 64))):
        assert np.array_equal(orc.gptq(w, S, sc, H, 0.01), _rtn(orc, w, S, sc))
    zero = np.zeros_like(w)
    _, X = _problem(5, cols=64)
    assert not orc.gptq(zero, S, sc, orc.full_hessian(X)).any()


def test_flip_takes_the_other_grid_neighbour(orc):
    """The flip option (used to follow a row past a near-tie resolved the other way): with a
    diagonal H there is no error feedback, so flipping column j changes only code j, to the
    grid neighbour on the side of |w_j| (one magnitude step, same sign, no signed zero);
    with a full H the columns before j are untouched and column j is that neighbour of the
    value it was rounded from. Saturated codes (|w| beyond 6 sS) keep their code."""
    w, X = _problem(9, rows=8, cols=64)
    S = orc.tensor_scale(w)
    sc = orc.scales_max(w, S)
    D = np.diag(np.random.default_rng(9).uniform(0.5, 3.0, 64))
    U = orc.gptq_factor(D, 0.01)
    plain = _unpack(orc.gptq(w, S, sc, U=U))
    for j in (0, 5, 31, 63):
        fl = np.full((8, 2), -1, np.int64)
        fl[:, 0] = j
        got = _unpack(orc.gptq(w, S, sc, U=U, flips=fl))
        others = np.delete(np.arange(64), j)
        assert np.array_equal(got[:, others], plain[:, others])
        for r in range(8):
            sS = orc.e4m3_value(int(sc[r, j // 16])) * float(S)
            k0, k1 = plain[r, j] & 7, got[r, j] & 7
            a, g0 = abs(float(w[r, j])), [0, .5, 1, 1.5, 2, 3, 4, 6][k0] * sS
            if a > g0 and k0 < 7:
                assert k1 == k0 + 1
            elif a < g0:
                assert k1 == k0 - 1
            else:
                assert k1 == k0
            if k1:
                assert (got[r, j] >> 3) == (1 if w[r, j] < 0 else 0)
            else:
                assert got[r, j] == 0
    H = orc.full_hessian(X)
    U = orc.gptq_factor(H, 0.01)
    base, v = orc.gptq(w, S, sc, U=U, return_v=True)
    base = _unpack(base)
    fl = np.full((8, 1), 20, np.int64)
    got, v2 = orc.gptq(w, S, sc, U=U, return_v=True, flips=fl)
    got = _unpack(got)
    assert np.array_equal(got[:, :20], base[:, :20]) and np.array_equal(v2[:, :21], v[:, :21])
    assert (got[:, 20] != base[:, 20]).any()


def _unpack(c):
    return np.stack([c & 15, c >> 4], -1).reshape(c.shape[0], -1)


def test_two_column_update_closed_form(orc):
    """Column 2 is rounded from w2 + (w1 - q1) H12 / H22 (damped H)."""
    rng = np.random.default_rng(6)
    S = np.float32(1e-3)
    byte = 60
    H = np.array([[3.0, 1.2], [1.2, 2.0]])
    lam = 0.01 * 2.5
    s = orc.e4m3_value(byte) * float(S)
    for _ in range(50):
        w = (rng.uniform(-5, 5, (1, 2)) * s).astype(np.float32)
        w16 = np.zeros((1, 16), np.float32)
        w16[0, :2] = w[0]
        Hf = np.eye(16)
        Hf[:2, :2] = H
        Hf[2:, 2:] *= 2.5  # keeps the mean diagonal at 2.5
        codes, v = orc.gptq(w16, S, np.array([[byte]], np.uint8), Hf, 0.01, return_v=True)
        q1 = orc.e2m1_value(codes[0, 0] & 15) * s
        v2 = float(w[0, 1]) + (float(w[0, 0]) - q1) * H[0, 1] / (H[1, 1] + lam)
        assert v[0, 1] == pytest.approx(v2, rel=1e-13, abs=1e-18)


def _obs_reference(w, S, sc, H, damp, orc):
    """GPTQ as repeated optimal updates: with columns < j fixed at their codes, the
    remaining weights move to minimise (w - v)^T Hd (w - v); solved directly per step."""
    n = w.shape[0]
    Hd = H + damp * np.trace(H) / n * np.eye(n)
    codes = np.zeros(n, np.int64)
    vals = np.zeros(n)
    q = np.zeros(n)
    for j in range(n):
        if j == 0:
            vj = float(w[0])
        else:
            delta = w[:j].astype(np.float64) - q[:j]
            dfree = -np.linalg.solve(Hd[j:, j:], Hd[j:, :j] @ delta)
            vj = float(w[j]) - dfree[0]
        byte = int(sc[j // 16])
        c = orc.e2m1_code_d(vj, byte, S)
        codes[j], vals[j] = c, vj
        q[j] = (-1 if c & 8 else 1) * orc.e2m1_value(c & 7) * orc.e4m3_value(byte) * float(S)
    return codes, vals


@pytest.mark.parametrize("seed", [7, 8, 9])
def test_matches_conditional_minimiser_formulation(orc, seed):
    w, X = _problem(seed, rows=4, cols=48)
    H = orc.full_hessian(X)
    S = orc.tensor_scale(w)
    sc = orc.scales_mse(w, S)
    codes, v = orc.gptq(w, S, sc, H, 0.01, return_v=True)
    unpacked = np.stack([codes & 15, codes >> 4], axis=-1).reshape(w.shape)
    for r in range(w.shape[0]):
        c_ref, v_ref = _obs_reference(w[r], S, sc[r], H, 0.01, orc)
        assert np.allclose(v[r], v_ref, rtol=1e-9, atol=1e-15)
        assert np.array_equal(unpacked[r], c_ref)


def test_lowers_output_error_against_plain_rounding(orc):
    w, X = _problem(10, rows=32, cols=128, tokens=512, corr=2.0)
    H = orc.full_hessian(X)
    S = orc.tensor_scale(w)
    sc = orc.scales_local_hessian(w, S, orc.block_hessian(X))
    rows, cols = w.shape
    deq = lambda c: orc.dequantize(c, sc, S, rows, cols).astype(np.float64)
    err = lambda c: np.einsum("ri,ij,rj->", deq(c) - w, H, deq(c) - w)
    e_gptq, e_rtn = err(orc.gptq(w, S, sc, H)), err(orc.quantize(w, S, sc))
    assert e_gptq < 0.9 * e_rtn, (e_gptq, e_rtn)


def test_power_of_two_scaling_of_h_changes_nothing(orc):
    w, X = _problem(11, rows=5, cols=64)
    H = orc.full_hessian(X)
    S = orc.tensor_scale(w)
    sc = orc.scales_max(w, S)
    c1, v1 = orc.gptq(w, S, sc, H, 0.01, return_v=True)
    c2, v2 = orc.gptq(w, S, sc, H * 4.0, 0.01, return_v=True)
    assert np.array_equal(c1, c2) and np.array_equal(v1, v2)
