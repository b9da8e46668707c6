"""Ridge fit of the per-layer maps, fp64 (oracle; test infrastructure only).

RidgeFill project page, "Method" step 2 and "Abstract": each late layer's input is
predicted from the split layer's state by a ridge regression fitted once in closed form
from one pass over calibration rows.  Notation: rows are token states x in R^{1 x d};
X is [n, d]; Y_l is [n, d] for late layer l; the prediction is y = x W_l + b_l.
"""
from __future__ import annotations

import numpy as np
import scipy.linalg
from scipy.linalg import lapack


class NotSPD(np.linalg.LinAlgError):
    """The regularised Gram is not positive definite; ``pivot`` is the 1-based order of the
    first leading minor that fails (LAPACK's convention)."""

    def __init__(self, pivot: int):
        super().__init__(f"regularised Gram not positive definite at pivot {pivot}")
        self.pivot = pivot


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def _cholesky_lower(A: np.ndarray) -> np.ndarray:
    L, info = lapack.dpotrf(A, lower=1, clean=1)
    if info > 0:
        raise NotSPD(int(info))
    if info < 0:
        raise ValueError(f"dpotrf argument {-info} invalid")
    return L


def _lambda_value(C: np.ndarray, lam: float, mode: str) -> float:
    if mode == "absolute":
        return float(lam)
    if mode == "rel_mean_diag":
        # KV-Lingo, Appendix B.2 "Protocol": ridge = factor x mean diagonal of the source Gram
        return float(lam) * float(np.mean(np.diag(C)))
    raise ValueError(mode)


def _solve_spd(A: np.ndarray, B: np.ndarray) -> np.ndarray:
    """A^-1 B for SPD A via Cholesky A = L L^T and two triangular solves."""
    L = _cholesky_lower(A)
    Z = scipy.linalg.solve_triangular(L, B, lower=True)
    return scipy.linalg.solve_triangular(L.T, Z, lower=False)


def fit(X, Y, lam: float, mode: str = "absolute"):
    """Ridge map with the intercept handled by mean-centring.

    X [n, d], Y [n, m] -> (W [d, m], b [m]) minimising
    ||(X - 1 mu_x) W - (Y - 1 mu_y)||_F^2 + lam ||W||_F^2, with b = mu_y - mu_x W.
    Centring is done on the rows first (two passes), so no cancellation enters C.
    """
    X = _f64(X)
    Y = _f64(Y)
    mu_x = X.mean(axis=0)
    mu_y = Y.mean(axis=0)
    Xc = X - mu_x
    Yc = Y - mu_y
    C = Xc.T @ Xc
    B = Xc.T @ Yc
    A = C + _lambda_value(C, lam, mode) * np.eye(C.shape[0])
    W = _solve_spd(A, B)
    b = mu_y - mu_x @ W
    return W, b


def gram_sums(X, Ys):
    """Raw one-pass statistics: (S_xx = X^T X, [S_xy_l = X^T Y_l], s_x = 1^T X, [s_y_l], n).

    These are the quantities a single streaming pass over calibration chunks can carry
    (RidgeFill "Method" step 2: one pass over calibration text)."""
    X = _f64(X)
    S_xx = X.T @ X
    s_x = X.sum(axis=0)
    S_xy = [X.T @ _f64(Y) for Y in Ys]
    s_y = [_f64(Y).sum(axis=0) for Y in Ys]
    return S_xx, S_xy, s_x, s_y, X.shape[0]


def fit_from_sums(S_xx, S_xy, s_x, s_y, n: int, lam: float, mode: str = "absolute"):
    """The same ridge map computed from the raw sums of ``gram_sums``.

    Centred Gram C = S_xx - s_x^T s_x / n, centred cross term B = S_xy - s_x^T s_y / n,
    then W = (C + lam I)^-1 B and b = s_y/n - (s_x/n) W."""
    S_xx = _f64(S_xx)
    s_x = _f64(s_x)
    C = S_xx - np.outer(s_x, s_x) / n
    A = C + _lambda_value(C, lam, mode) * np.eye(C.shape[0])
    L = _cholesky_lower(A)
    out = []
    for Sxy, sy in zip(S_xy, s_y):
        B = _f64(Sxy) - np.outer(s_x, _f64(sy)) / n
        Z = scipy.linalg.solve_triangular(L, B, lower=True)
        W = scipy.linalg.solve_triangular(L.T, Z, lower=False)
        b = _f64(sy) / n - (s_x / n) @ W
        out.append((W, b))
    return out


def solve_columns_from_data(X, Y_cols, lam: float, mode: str = "absolute"):
    """Selected output columns of the ridge map, from the data.

    Column j of W depends only on column j of Y, so a sample of columns can be checked at
    full size: X [n, d], Y_cols [n, k] -> (W_cols [d, k], b_cols [k])."""
    return fit(X, Y_cols, lam, mode)


def stationarity_residual(X, Y, W, lam: float, mode: str = "absolute") -> float:
    """How far W is from solving the ridge normal equations on the centred rows: with
    C = X~^T X~ and B = X~^T Y~, max |(C + lam I) W - B| / max |B| (0 for the exact map).
    The ridge map is the stationary point of the objective, where X~^T (X~ W - Y~) + lam W = 0;
    this is that gradient, scaled by the cross moments."""
    X = _f64(X)
    Y = _f64(Y)
    Xc = X - X.mean(axis=0)
    Yc = Y - Y.mean(axis=0)
    C = Xc.T @ Xc
    B = Xc.T @ Yc
    A = C + _lambda_value(C, lam, mode) * np.eye(C.shape[0])
    return float(np.max(np.abs(A @ _f64(W) - B)) / np.max(np.abs(B)))


def stationarity_residual_from_sums(S_xx, S_xy, s_x, s_y, n: int, W, lam: float, mode: str = "absolute") -> float:
    """The same residual with C and B centred from raw one-pass sums (as ``fit_from_sums``):
    C = S_xx - s_x^T s_x / n, B = S_xy - s_x^T s_y / n.  S_xx must be the full symmetric matrix."""
    S_xx = _f64(S_xx)
    s_x = _f64(s_x)
    C = S_xx - np.outer(s_x, s_x) / n
    B = _f64(S_xy) - np.outer(s_x, _f64(s_y)) / n
    A = C + _lambda_value(C, lam, mode) * np.eye(C.shape[0])
    return float(np.max(np.abs(A @ _f64(W) - B)) / np.max(np.abs(B)))


def ridge_objective(X, Y, W, lam: float) -> float:
    """The ridge objective on centred rows, used to check optimality by perturbation."""
    X = _f64(X)
    Y = _f64(Y)
    Xc = X - X.mean(axis=0)
    Yc = Y - Y.mean(axis=0)
    R = Xc @ _f64(W) - Yc
    return float(np.sum(R * R) + lam * np.sum(_f64(W) ** 2))


def fit_pinv(X, Y, lam: float = 0.0, rel_tol: float = 1e-8, mode: str = "absolute"):
    """The map by the symmetric eigendecomposition route (KV-Lingo page, appendix on the
    training procedure, "Stage 1": the per-layer normal equations are solved once by symmetric
    eigendecomposition, eigenvalues below a relative tolerance of 1e-8 counting as zero).  A = X~^T X~ + lam I = V diag(mu) V^T;
    A^+ keeps 1/mu_i for mu_i > rel_tol * max(mu) and zero otherwise; W = A^+ X~^T Y~ and
    b = mean(Y) - mean(X) W.  For a regular A this is the ridge map of ``fit``; for a singular
    one it is the minimum-norm least-squares map."""
    X = _f64(X)
    Y = _f64(Y)
    mu_x = X.mean(axis=0)
    mu_y = Y.mean(axis=0)
    Xc = X - mu_x
    Yc = Y - mu_y
    C = Xc.T @ Xc
    A = C + _lambda_value(C, lam, mode) * np.eye(C.shape[0])
    mu, V = np.linalg.eigh(A)
    keep = mu > rel_tol * np.max(mu)
    inv = np.where(keep, 1.0 / np.where(keep, mu, 1.0), 0.0)
    W = (V * inv) @ V.T @ (Xc.T @ Yc)
    return W, mu_y - mu_x @ W
