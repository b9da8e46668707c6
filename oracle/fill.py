"""Late-layer cache fill, fp64 (oracle; test infrastructure only).

RidgeFill project page, "Method" steps 2-3 and Figure 2(b): for every filled prompt row and
every late layer, predict the layer's input from the split layer's state with that layer's
map, then let the layer's own projections write its K/V cache from the prediction.  The
KV-Lingo page (section 3.1, "Rotation and normalisation"; section 2, notation) fixes the
pre-norm storing order: the predicted input is normalised, projected, and only keys are
rotated by their token's position before they are stored.

Notation: x in R^{1 x d} is a token's split-layer state; for late layer l the stored weights
are W_l [d, d], b_l [d], gamma_l [d], W_K^l [d, H*d_h], W_V^l [d, H*d_h] (x-times-matrix
convention, head-major output columns: column g*d_h + j is head g, dim j).
"""
from __future__ import annotations

import numpy as np


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def rope_inverse_frequencies(head_dim: int, base: float) -> np.ndarray:
    """theta_i = base^(-2i/d_h) for i in [0, d_h/2)."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * i / head_dim)


def rope_rotate(k, positions, base: float) -> np.ndarray:
    """Rotate-half RoPE on per-head vectors.

    k [T, H, d_h]; positions [T] (absolute, 0-based).  The pair (i, i + d_h/2) of every head
    is rotated by the angle pos * theta_i:
        (a, c) -> (a cos - c sin, c cos + a sin)."""
    k = _f64(k)
    half = k.shape[-1] // 2
    phi = _f64(positions)[:, None] * rope_inverse_frequencies(k.shape[-1], base)[None, :]
    cos = np.cos(phi)[:, None, :]
    sin = np.sin(phi)[:, None, :]
    a = k[..., :half]
    c = k[..., half:]
    return np.concatenate([a * cos - c * sin, c * cos + a * sin], axis=-1)


def rmsnorm(h, gamma, eps: float) -> np.ndarray:
    """u = h / sqrt(mean_j h_j^2 + eps) * gamma, row by row."""
    h = _f64(h)
    r = 1.0 / np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + eps)
    return h * r * _f64(gamma)


def fill_layer(X, W, b, gamma, W_K, W_V, positions, n_kv_heads: int, head_dim: int,
               eps: float, base: float, k_norm=None, k_norm_eps: float = 1e-6):
    """K and V rows of one late layer for the token states X [T, d].

    h = x W + b (predicted input); u = RMSNorm(h) * gamma; k = u W_K, v = u W_V; with
    ``k_norm`` (gamma_k [d_h]) each head of k is RMS-normalised (KV-Lingo page, section 2: some
    models normalise keys per head before rotating them); RoPE on k.
    Returns (K, V), each [T, H, d_h] fp64."""
    X = _f64(X)
    H = X @ _f64(W) + _f64(b)
    U = rmsnorm(H, gamma, eps)
    K = (U @ _f64(W_K)).reshape(X.shape[0], n_kv_heads, head_dim)
    V = (U @ _f64(W_V)).reshape(X.shape[0], n_kv_heads, head_dim)
    if k_norm is not None:
        K = rmsnorm(K, k_norm, k_norm_eps)
    return rope_rotate(K, positions, base), V


def fill(X, t0: int, t1: int, pos0: int, layers, n_kv_heads: int, head_dim: int,
         eps: float, base: float, k_norm_eps: float = 1e-6):
    """Fill token rows [t0, t1) of every listed layer.

    X holds the split-layer states of tokens t0..t1-1 (row i is token t0 + i); token t sits
    at RoPE position pos0 + t.  ``layers`` is a sequence of (W, b, gamma, W_K, W_V), or of
    (W, b, gamma, W_K, W_V, gamma_k) for layers that normalise keys per head.
    Returns a list of (K, V) per layer, each [t1 - t0, H, d_h]."""
    X = _f64(X)
    if X.shape[0] != t1 - t0:
        raise ValueError("X must hold exactly the rows [t0, t1)")
    positions = pos0 + np.arange(t0, t1, dtype=np.float64)
    out = []
    for lw in layers:
        kn = lw[5] if len(lw) > 5 else None
        out.append(fill_layer(X, *lw[:5], positions, n_kv_heads, head_dim, eps, base, kn, k_norm_eps))
    return out
