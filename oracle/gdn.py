"""Gated DeltaNet state update over a token range, fp64 (oracle; test infrastructure only).

RidgeFill project page, "Method" step 3 and Figure 2(b): each late layer's own projections
run on the predicted input, and on a Gated DeltaNet layer so does its state update.  The page
does not write the update out; it is the published Gated DeltaNet recurrence (Yang, Kautz and
Hatamizadeh, "Gated Delta Networks: Improving Mamba2 with Delta Rule", 2024), per head:

    S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   alpha_t = exp(g_t),

with the state S in R^{d_v x d_k}, the token's key k_t (L2-normalised by the layer, as that
paper does before the update) and value v_t, the gate g_t <= 0 and the write strength
beta_t in [0, 1].  Written here as the plain sequential recurrence, one token after the other.
Parity of this function against the pages is unpinned (the pages give no update, no worked
value and no gate law); its pins are the recurrence's own closed forms (see the tests).
"""
from __future__ import annotations

import numpy as np


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def l2_normalise(k, eps: float = 1e-6) -> np.ndarray:
    """k / sqrt(sum k^2 + eps) over the last axis (eps inside the root)."""
    k = _f64(k)
    return k / np.sqrt(np.sum(k * k, axis=-1, keepdims=True) + eps)


def gdn_state(K, V, g, beta, S0=None, normalise_k: bool = False, eps: float = 1e-6) -> np.ndarray:
    """The state after tokens 0..T-1.

    K [T, H, d_k], V [T, H, d_v], g [T, H] (log decay), beta [T, H]; S0 [H, d_v, d_k] or None
    (zeros).  With ``normalise_k`` the keys are L2-normalised per head first.
    Returns S [H, d_v, d_k]."""
    K = _f64(K)
    V = _f64(V)
    g = _f64(g)
    beta = _f64(beta)
    if normalise_k:
        K = l2_normalise(K, eps)
    T, H, dk = K.shape
    dv = V.shape[2]
    S = np.zeros((H, dv, dk)) if S0 is None else _f64(S0).copy()
    for t in range(T):
        for h in range(H):
            k = K[t, h]
            a = np.exp(g[t, h])
            b = beta[t, h]
            # S (I - b k k^T) = S - b (S k) k^T
            S[h] = a * (S[h] - b * np.outer(S[h] @ k, k)) + b * np.outer(V[t, h], k)
    return S
