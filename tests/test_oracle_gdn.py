"""Pins of the oracle's Gated DeltaNet state update (the published recurrence the RidgeFill
project page names in "Method" step 3): closed forms of the recurrence, a hand-worked token,
the delta rule's exact-write and overwrite properties, its reading as one gradient step, and
chunked continuation.  Against the pages themselves its parity is unpinned."""
import numpy as np
import pytest

import oracle


def test_hand_worked_token():
    # S0 = [[1, 2]], k = (0.6, 0.8) (unit), v = 3, alpha = 0.5, beta = 0.5:
    # S0 k = 2.2; S0 - 0.5 * 2.2 k^T = (0.34, 1.12); * 0.5 = (0.17, 0.56); + 0.5 * 3 k^T = (0.9, 1.2)
    S = oracle.gdn_state(np.array([[[0.6, 0.8]]]), np.array([[[3.0]]]), np.log([[0.5]]), np.array([[0.5]]),
                         S0=np.array([[[1.0, 2.0]]]))
    assert np.allclose(S, [[[1.07, 1.76]]], rtol=0, atol=1e-14)


def test_no_write_no_decay_and_decay_only():
    rng = np.random.default_rng(0)
    T, H, dk, dv = 7, 3, 5, 4
    K, V = rng.standard_normal((T, H, dk)), rng.standard_normal((T, H, dv))
    S0 = rng.standard_normal((H, dv, dk))
    zeros = np.zeros((T, H))
    assert np.array_equal(oracle.gdn_state(K, V, zeros, zeros, S0), S0)
    g = -rng.random((T, H))
    S = oracle.gdn_state(K, V, g, zeros, S0)
    assert np.allclose(S, np.exp(g.sum(0))[:, None, None] * S0, rtol=1e-14, atol=0)


def test_one_token_from_zero_state():
    rng = np.random.default_rng(1)
    K, V = rng.standard_normal((1, 2, 6)), rng.standard_normal((1, 2, 3))
    beta = np.array([[0.3, 0.9]])
    S = oracle.gdn_state(K, V, np.array([[-0.2, -1.0]]), beta)
    for h in range(2):
        assert np.allclose(S[h], beta[0, h] * np.outer(V[0, h], K[0, h]), rtol=1e-15, atol=1e-15)


def test_delta_rule_writes_and_overwrites_exactly():
    # beta = 1 and a unit key: after the token the state maps the key to its value exactly,
    # whatever it held and however it decayed; orthonormal keys store side by side
    rng = np.random.default_rng(2)
    dk, dv = 8, 5
    Q, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    keys = Q[:, :4].T                                     # 4 orthonormal keys
    vals = rng.standard_normal((4, dv))
    K = keys[:, None, :]
    V = vals[:, None, :]
    S = oracle.gdn_state(K, V, np.zeros((4, 1)), np.ones((4, 1)), S0=rng.standard_normal((1, dv, dk)) * 0)
    for i in range(4):
        assert np.allclose(S[0] @ keys[i], vals[i], atol=1e-13)
    assert np.allclose(S[0], vals.T @ keys, atol=1e-13)
    # the same key written twice: the second value replaces the first
    v2 = rng.standard_normal(dv)
    S2 = oracle.gdn_state(np.concatenate([K, K[:1]]), np.concatenate([V, v2[None, None, :]]),
                          np.concatenate([np.zeros((4, 1)), [[-0.7]]]), np.ones((5, 1)))
    assert np.allclose(S2[0] @ keys[0], v2, atol=1e-13)


def test_update_is_one_gradient_step_on_the_decayed_state():
    # S_t = S' - beta dL/dS at S' = alpha S_{t-1}, L(S) = |S k - v|^2 / 2 (gradient taken by
    # central differences, independently of the recurrence's algebra)
    rng = np.random.default_rng(3)
    dk, dv = 4, 3
    S0 = rng.standard_normal((dv, dk))
    k, v = rng.standard_normal(dk), rng.standard_normal(dv)
    a, b = 0.8, 0.45
    Sp = a * S0
    L = lambda S: 0.5 * np.sum((S @ k - v) ** 2)
    grad = np.zeros_like(Sp)
    h = 1e-6
    for i in range(dv):
        for j in range(dk):
            E = np.zeros_like(Sp)
            E[i, j] = h
            grad[i, j] = (L(Sp + E) - L(Sp - E)) / (2 * h)
    S = oracle.gdn_state(k[None, None, :], v[None, None, :], np.log([[a]]), np.array([[b]]), S0=S0[None])
    assert np.allclose(S[0], Sp - b * grad, atol=1e-8)


def test_chunked_continuation_and_key_normalisation():
    rng = np.random.default_rng(4)
    T, H, dk, dv = 23, 2, 6, 5
    K, V = rng.standard_normal((T, H, dk)), rng.standard_normal((T, H, dv))
    g, beta = -rng.random((T, H)), rng.random((T, H))
    full = oracle.gdn_state(K, V, g, beta, normalise_k=True)
    for cut in (1, 9, 22):
        first = oracle.gdn_state(K[:cut], V[:cut], g[:cut], beta[:cut], normalise_k=True)
        both = oracle.gdn_state(K[cut:], V[cut:], g[cut:], beta[cut:], S0=first, normalise_k=True)
        assert np.allclose(both, full, rtol=1e-13, atol=1e-13)
    Kn = K / np.sqrt(np.sum(K * K, axis=-1, keepdims=True) + 1e-6)
    assert np.allclose(oracle.gdn_state(Kn, V, g, beta), full, rtol=1e-13, atol=1e-13)
    # normalised keys, gates in (0, 1]: the update is a contraction plus a bounded write, so the
    # state stays bounded by the largest value norm over (1 - decay) ... checked loosely
    assert np.all(np.isfinite(full)) and np.max(np.abs(full)) < 50
