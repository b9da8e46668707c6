"""Pins of the oracle's ridge fit against what the mathematics fixes (CPU only).

Each test checks the oracle against something other than its own formula: a hand-solved
case in exact fractions, exact rational brute force, planted recovery, an SVD least-squares
route, an eigendecomposition pseudo-inverse route, optimality by perturbation, limits and
invariances.  A dropped centring term, a transposed operand, a wrong lambda placement or a
wrong triangular solve each fail at least one of them (see test_oracle_mutations.py).
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle


def _rng(seed):
    return np.random.default_rng(seed)


def test_ridge_1d_solved_by_hand():
    # x = [1,2,3,4], y = [2,4,5,9], lambda = 1.
    # centred x = [-3/2,-1/2,1/2,3/2], centred y = [-3,-1,0,4]
    # sum x~y~ = 11, sum x~^2 = 5  ->  W = 11/6,  b = 5 - (5/2)(11/6) = 5/12
    X = np.array([[1.0], [2.0], [3.0], [4.0]])
    Y = np.array([[2.0], [4.0], [5.0], [9.0]])
    W, b = oracle.fit(X, Y, 1.0)
    assert W[0, 0] == pytest.approx(11 / 6, rel=1e-15)
    assert b[0] == pytest.approx(5 / 12, rel=1e-14)


def _exact_ridge(Xi, Yi, lam: Fraction):
    """Exact rational ridge with intercept by Gauss-Jordan elimination (no Cholesky)."""
    n, d = len(Xi), len(Xi[0])
    m = len(Yi[0])
    mx = [sum(Fraction(Xi[r][j]) for r in range(n)) / n for j in range(d)]
    my = [sum(Fraction(Yi[r][j]) for r in range(n)) / n for j in range(m)]
    Xc = [[Fraction(Xi[r][j]) - mx[j] for j in range(d)] for r in range(n)]
    Yc = [[Fraction(Yi[r][j]) - my[j] for j in range(m)] for r in range(n)]
    A = [[sum(Xc[r][i] * Xc[r][j] for r in range(n)) + (lam if i == j else 0)
          for j in range(d)] for i in range(d)]
    B = [[sum(Xc[r][i] * Yc[r][j] for r in range(n)) for j in range(m)] for i in range(d)]
    # augmented [A | B], full Gauss-Jordan with exact pivots
    M = [A[i] + B[i] for i in range(d)]
    for c in range(d):
        p = next(r for r in range(c, d) if M[r][c] != 0)
        M[c], M[p] = M[p], M[c]
        pv = M[c][c]
        M[c] = [v / pv for v in M[c]]
        for r in range(d):
            if r != c and M[r][c] != 0:
                f = M[r][c]
                M[r] = [vr - f * vc for vr, vc in zip(M[r], M[c])]
    W = [[M[i][d + j] for j in range(m)] for i in range(d)]
    b = [my[j] - sum(mx[i] * W[i][j] for i in range(d)) for j in range(m)]
    return W, b


@pytest.mark.parametrize("d,n,m,seed", [(3, 7, 2, 0), (6, 11, 3, 1), (16, 24, 2, 2)])
def test_bruteforce_exact_rational(d, n, m, seed):
    rng = _rng(seed)
    Xi = rng.integers(-5, 6, size=(n, d)).tolist()
    Yi = rng.integers(-5, 6, size=(n, m)).tolist()
    lam = Fraction(3, 2)
    W_ex, b_ex = _exact_ridge(Xi, Yi, lam)
    W, b = oracle.fit(np.array(Xi, float), np.array(Yi, float), 1.5)
    W_ex = np.array([[float(v) for v in row] for row in W_ex])
    b_ex = np.array([float(v) for v in b_ex])
    assert np.max(np.abs(W - W_ex)) <= 1e-12 * max(1.0, np.max(np.abs(W_ex)))
    assert np.max(np.abs(b - b_ex)) <= 1e-12 * max(1.0, np.max(np.abs(b_ex)))


def test_planted_recovery_and_intercept():
    rng = _rng(3)
    n, d, m = 300, 24, 10
    X = rng.standard_normal((n, d))
    A = rng.standard_normal((d, m))
    c = rng.standard_normal(m)
    Y = X @ A + c
    Xc = X - X.mean(0)
    lam = 1e-12 * np.trace(Xc.T @ Xc) / d
    W, b = oracle.fit(X, Y, lam)
    assert np.max(np.abs(W - A)) / np.max(np.abs(A)) <= 1e-10
    assert np.max(np.abs(b - c)) / np.max(np.abs(c)) <= 1e-10


def test_svd_least_squares_route():
    # ridge == ordinary least squares on rows [X~; sqrt(lam) I] against [Y~; 0]
    rng = _rng(4)
    n, d, m, lam = 80, 12, 5, 3.7
    X = rng.standard_normal((n, d)) * np.linspace(0.2, 4.0, d)
    Y = rng.standard_normal((n, m)) + X[:, :m]
    W, b = oracle.fit(X, Y, lam)
    Xc = X - X.mean(0)
    Yc = Y - Y.mean(0)
    Xa = np.vstack([Xc, np.sqrt(lam) * np.eye(d)])
    Ya = np.vstack([Yc, np.zeros((d, m))])
    W_ls = np.linalg.lstsq(Xa, Ya, rcond=None)[0]
    assert np.max(np.abs(W - W_ls)) <= 1e-12 * np.max(np.abs(W_ls))
    assert np.allclose(b, Y.mean(0) - X.mean(0) @ W_ls, rtol=0, atol=1e-12)


def test_eig_pseudo_inverse_route_small_lambda():
    # KV-Lingo Appendix stage 1: normal equations solved by symmetric eigendecomposition,
    # eigenvalues below 1e-8 relative treated as zero.  On full-rank data, lambda -> 0 ridge
    # must agree with it.
    rng = _rng(5)
    n, d, m = 500, 20, 6
    X = rng.standard_normal((n, d))
    Y = rng.standard_normal((n, m))
    W, _ = oracle.fit(X, Y, 1e-9)
    Xc = X - X.mean(0)
    Yc = Y - Y.mean(0)
    evals, evecs = np.linalg.eigh(Xc.T @ Xc)
    keep = evals > 1e-8 * evals.max()
    inv = (evecs[:, keep] / evals[keep]) @ evecs[:, keep].T
    W_pinv = inv @ (Xc.T @ Yc)
    assert np.max(np.abs(W - W_pinv)) <= 1e-8 * np.max(np.abs(W_pinv))


def test_optimality_by_perturbation():
    rng = _rng(6)
    n, d, m, lam = 60, 9, 4, 2.5
    X = rng.standard_normal((n, d))
    Y = rng.standard_normal((n, m))
    W, _ = oracle.fit(X, Y, lam)
    J0 = oracle.ridge_objective(X, Y, W, lam)
    for k in range(20):
        D = rng.standard_normal(W.shape)
        for eps in (1e-3, 1e-1):
            assert oracle.ridge_objective(X, Y, W + eps * D, lam) > J0
    # first-order: the directional derivative vanishes
    D = rng.standard_normal(W.shape)
    h = 1e-4
    g = (oracle.ridge_objective(X, Y, W + h * D, lam) - oracle.ridge_objective(X, Y, W - h * D, lam)) / (2 * h)
    assert abs(g) <= 1e-6 * J0


def test_large_lambda_limit():
    rng = _rng(7)
    X = rng.standard_normal((50, 8))
    Y = rng.standard_normal((50, 3))
    lam = 1e10
    W, _ = oracle.fit(X, Y, lam)
    Xc = X - X.mean(0)
    B = Xc.T @ (Y - Y.mean(0))
    assert np.max(np.abs(lam * W - B)) <= 1e-7 * np.max(np.abs(B))


def test_column_shift_and_row_permutation_invariance():
    rng = _rng(8)
    X = rng.standard_normal((70, 10))
    Y = rng.standard_normal((70, 4))
    W, b = oracle.fit(X, Y, 0.5)
    c = rng.standard_normal(10) * 5
    W2, b2 = oracle.fit(X + c, Y, 0.5)
    assert np.allclose(W2, W, rtol=0, atol=1e-12)
    assert np.allclose(b2, b - c @ W, rtol=0, atol=1e-12)
    p = rng.permutation(70)
    W3, b3 = oracle.fit(X[p], Y[p], 0.5)
    assert np.allclose(W3, W, rtol=0, atol=1e-12) and np.allclose(b3, b, rtol=0, atol=1e-12)


def test_chunked_sums_equal_one_shot_fit():
    rng = _rng(9)
    X = rng.standard_normal((120, 10)) + 0.3
    Ys = [rng.standard_normal((120, 10)) + X * 0.5, rng.standard_normal((120, 10))]
    one = oracle.gram_sums(X, Ys)
    parts = [oracle.gram_sums(X[a:a + 40], [Y[a:a + 40] for Y in Ys]) for a in (0, 40, 80)]
    S_xx = sum(p[0] for p in parts)
    S_xy = [sum(p[1][l] for p in parts) for l in range(2)]
    s_x = sum(p[2] for p in parts)
    s_y = [sum(p[3][l] for p in parts) for l in range(2)]
    n = sum(p[4] for p in parts)
    assert n == one[4] == 120
    assert np.allclose(S_xx, one[0], rtol=1e-13, atol=1e-12)
    fits = oracle.fit_from_sums(S_xx, S_xy, s_x, s_y, n, 0.2)
    for (W, b), Y in zip(fits, Ys):
        W0, b0 = oracle.fit(X, Y, 0.2)
        assert np.allclose(W, W0, rtol=0, atol=1e-11) and np.allclose(b, b0, rtol=0, atol=1e-11)


def test_not_spd_reports_pivot():
    rng = _rng(10)
    X = rng.standard_normal((40, 6))
    X[:, 3] = 0.0                     # constant channel: centred Gram row 3 is exactly zero
    Y = rng.standard_normal((40, 2))
    with pytest.raises(oracle.NotSPD) as e:
        oracle.fit(X, Y, 0.0)
    assert e.value.pivot == 4         # 1-based order of the first failing leading minor
    S = oracle.gram_sums(X, [Y])
    with pytest.raises(oracle.NotSPD):
        oracle.fit_from_sums(*S, 0.0)
    oracle.fit(X, Y, 1e-3)            # any lambda > 0 restores positive definiteness


def test_relative_lambda_is_scale_free():
    # lambda relative to the mean Gram diagonal: scaling X and Y by c leaves W unchanged,
    # while an absolute lambda does not.
    rng = _rng(11)
    X = rng.standard_normal((60, 8))
    Y = rng.standard_normal((60, 3))
    W1, _ = oracle.fit(X, Y, 1e-1, mode="rel_mean_diag")
    W2, _ = oracle.fit(7.0 * X, 7.0 * Y, 1e-1, mode="rel_mean_diag")
    assert np.allclose(W1, W2, rtol=0, atol=1e-12)
    Wa, _ = oracle.fit(X, Y, 5.0)
    Wb, _ = oracle.fit(7.0 * X, 7.0 * Y, 5.0)
    assert not np.allclose(Wa, Wb, rtol=0, atol=1e-6)


def test_pinv_route_regular_equals_cholesky_fit():
    # a regular system: the eigendecomposition route and the Cholesky route agree
    rng = np.random.default_rng(21)
    X = rng.standard_normal((300, 12)) * np.linspace(0.3, 3, 12) + 1.0
    Y = X @ rng.standard_normal((12, 5)) + rng.standard_normal((300, 5))
    for lam in (0.0, 1e-2, 10.0):
        W1, b1 = oracle.fit(X, Y, lam)
        W2, b2 = oracle.fit_pinv(X, Y, lam)
        assert np.max(np.abs(W1 - W2)) <= 1e-10 * np.max(np.abs(W1))
        assert np.max(np.abs(b1 - b2)) <= 1e-10 * max(1.0, np.max(np.abs(b1)))


def test_pinv_route_rank_deficient_is_minimum_norm_least_squares():
    # duplicated and zero-variance columns make X~^T X~ singular: the route gives the
    # minimum-norm least-squares map, as an SVD solver does (numpy.linalg.lstsq, an independent
    # library route), and it leaves the null space of X~ out of W
    rng = np.random.default_rng(22)
    n = 400
    base = rng.standard_normal((n, 6))
    X = np.hstack([base, base[:, :2], np.full((n, 1), 3.0), base[:, 3:4] * 2.0])   # rank 6 of 10
    Y = base @ rng.standard_normal((6, 4)) + 0.1 * rng.standard_normal((n, 4))
    W, b = oracle.fit_pinv(X, Y, 0.0)
    Xc, Yc = X - X.mean(0), Y - Y.mean(0)
    W_ls = np.linalg.lstsq(Xc, Yc, rcond=1e-10)[0]
    assert np.max(np.abs(W - W_ls)) <= 1e-9 * np.max(np.abs(W_ls))
    assert np.allclose(b, Y.mean(0) - X.mean(0) @ W_ls, rtol=0, atol=1e-9)
    # null-space directions of X~ (the duplicate differences, the constant column) get nothing
    null = np.zeros((10, 4))
    null[0, 0], null[6, 0] = 1.0, -1.0
    null[1, 1], null[7, 1] = 1.0, -1.0
    null[8, 2] = 1.0
    null[3, 3], null[9, 3] = 2.0, -1.0
    assert np.allclose(Xc @ null, 0.0, atol=1e-12)
    assert np.max(np.abs(null.T @ W)) <= 1e-9 * np.max(np.abs(W))


def test_stationarity_residual_hand_worked_and_limits():
    # one feature, three rows: X~ = (-1, 0, 1), Y~ = (-7/3, -1/3, 8/3), so C = 2, B = 5; with
    # lambda = 1, A = 3 and the residual of w is |3 w - 5| / 5 (0.4 at w = 1, 0 at w = 5/3)
    X = np.array([[1.0], [2.0], [3.0]])
    Y = np.array([[2.0], [4.0], [7.0]])
    assert abs(oracle.stationarity_residual(X, Y, np.array([[1.0]]), 1.0) - 0.4) <= 1e-15
    assert oracle.stationarity_residual(X, Y, np.array([[5.0 / 3.0]]), 1.0) <= 1e-15
    # W = 0 leaves all of B
    rng = np.random.default_rng(3)
    X = rng.standard_normal((200, 6))
    Y = X @ rng.standard_normal((6, 4)) + 0.1 * rng.standard_normal((200, 4))
    assert oracle.stationarity_residual(X, Y, np.zeros((6, 4)), 0.5) == 1.0
    # the fitted map is stationary to fp64 rounding (<= 1e-12)
    W, _ = oracle.fit(X, Y, 0.5)
    assert oracle.stationarity_residual(X, Y, W, 0.5) <= 1e-12
    # one entry moved by delta: the residual is delta times the largest entry of that row of A
    Xc = X - X.mean(0)
    A = Xc.T @ Xc + 0.5 * np.eye(6)
    B = Xc.T @ (Y - Y.mean(0))
    W2 = W.copy()
    W2[2, 1] += 1e-3
    want = 1e-3 * np.max(np.abs(A[:, 2])) / np.max(np.abs(B))
    assert abs(oracle.stationarity_residual(X, Y, W2, 0.5) - want) <= 1e-12
    # a transposed map (a plausible layout mistake) is far from stationary
    Ws, _ = oracle.fit(X, X @ rng.standard_normal((6, 6)), 0.5)
    assert oracle.stationarity_residual(X, X @ Ws, Ws.T, 0.5) > 1e-2


def test_stationarity_residual_from_sums_equals_data_route():
    rng = np.random.default_rng(4)
    X = rng.standard_normal((300, 8)) + 2.0
    Y = X @ rng.standard_normal((8, 5)) + rng.standard_normal((300, 5))
    W = rng.standard_normal((8, 5))
    S_xx, S_xy, s_x, s_y, n = oracle.gram_sums(X, [Y])
    for lam, mode in ((0.3, "absolute"), (1e-2, "rel_mean_diag")):
        a = oracle.stationarity_residual(X, Y, W, lam, mode)
        b = oracle.stationarity_residual_from_sums(S_xx, S_xy[0], s_x, s_y[0], n, W, lam, mode)
        assert abs(a - b) <= 1e-12 * max(1.0, a)
