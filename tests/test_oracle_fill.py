"""Pins of the oracle's cache fill against closed forms and invariants (CPU only)."""
import math

import numpy as np
import pytest

import oracle


def test_hand_worked_rmsnorm_rope():
    # d = 4, one head of d_h = 4, identity map, gamma = 1, eps = 0, W_K = W_V = I,
    # base 100, token at position 1.
    # x = [3, 4, 0, 0]: mean h^2 = 25/4, so u = x / 2.5 = [1.2, 1.6, 0, 0]
    # theta = [100^0, 100^-0.5] = [1, 0.1]; pairs (0,2) turn by 1 rad, (1,3) by 0.1 rad.
    I = np.eye(4)
    K, V = oracle.fill_layer(np.array([[3.0, 4.0, 0.0, 0.0]]), I, np.zeros(4), np.ones(4),
                             I, I, np.array([1.0]), 1, 4, 0.0, 100.0)
    expect_k = [1.2 * math.cos(1.0), 1.6 * math.cos(0.1), 1.2 * math.sin(1.0), 1.6 * math.sin(0.1)]
    assert np.allclose(K[0, 0], expect_k, rtol=0, atol=1e-15)
    assert np.allclose(V[0, 0], [1.2, 1.6, 0.0, 0.0], rtol=0, atol=1e-15)


def test_rmsnorm_epsilon_inside_root():
    h = np.array([[1.0, 2.0, 3.0, 4.0]])          # mean square 7.5
    u = oracle.rmsnorm(h, np.ones(4), 0.5)
    assert np.allclose(u, h / math.sqrt(8.0), rtol=0, atol=1e-15)
    g = np.array([1.0, -2.0, 0.5, 3.0])
    assert np.allclose(oracle.rmsnorm(h, g, 0.5), h / math.sqrt(8.0) * g, rtol=0, atol=1e-15)


def _rope_complex(k, positions, base):
    # independent route: pair (i, i+h) as the complex number a + i c, times e^{i pos theta}
    half = k.shape[-1] // 2
    theta = np.array([base ** (-(2.0 * i) / k.shape[-1]) for i in range(half)])
    z = (k[..., :half] + 1j * k[..., half:]) * np.exp(1j * positions[:, None, None] * theta)
    return np.concatenate([z.real, z.imag], axis=-1)


def test_rope_matches_complex_rotation_and_invariants():
    rng = np.random.default_rng(0)
    k = rng.standard_normal((9, 3, 16))
    pos = np.array([0, 1, 2, 7, 100, 4095, 65536, 131071, 3.0])
    base = 5e5
    r = oracle.rope_rotate(k, pos, base)
    assert np.allclose(r, _rope_complex(k, pos, base), rtol=0, atol=1e-12)
    # position 0 is the identity; every pair keeps its norm
    assert np.array_equal(r[0], k[0])
    half = 8
    n0 = k[..., :half] ** 2 + k[..., half:] ** 2
    n1 = r[..., :half] ** 2 + r[..., half:] ** 2
    assert np.allclose(n0, n1, rtol=1e-12, atol=0)
    # <RoPE(q, m), RoPE(k, n)> depends only on m - n
    q = rng.standard_normal((1, 1, 16))
    kk = rng.standard_normal((1, 1, 16))
    dots = []
    for m, n in [(5, 2), (1003, 1000), (70003, 70000)]:
        a = oracle.rope_rotate(q, np.array([m]), base)
        b = oracle.rope_rotate(kk, np.array([n]), base)
        dots.append(float(np.sum(a * b)))
    assert np.allclose(dots, dots[0], rtol=1e-9, atol=1e-12)


def _rand_layer(rng, d, kvw, identity=False):
    W = np.eye(d) if identity else np.eye(d) + 0.1 * rng.standard_normal((d, d))
    b = np.zeros(d) if identity else 0.1 * rng.standard_normal(d)
    g = 1.0 + 0.1 * rng.standard_normal(d)
    return W, b, g, 0.2 * rng.standard_normal((d, kvw)), 0.2 * rng.standard_normal((d, kvw))


def test_identity_fill_equals_exact_recompute():
    # RidgeFill project page, reference study: the identity fill uses the split layer's
    # state as every late layer's input.  Then the fill must equal an independent exact
    # recompute of the layer's K/V from x.
    rng = np.random.default_rng(1)
    d, H, dh, T = 32, 2, 8, 11
    X = rng.standard_normal((T, d)) * 3.0
    W, b, g, Wk, Wv = _rand_layer(rng, d, H * dh, identity=True)
    (K, V), = oracle.fill(X, 5, 5 + T, 17, [(W, b, g, Wk, Wv)], H, dh, 1e-6, 1e4)
    u = X / np.sqrt((X ** 2).mean(-1, keepdims=True) + 1e-6) * g
    pos = 17 + np.arange(5, 5 + T, dtype=float)
    K_ref = _rope_complex((u @ Wk).reshape(T, H, dh), pos, 1e4)
    assert np.allclose(K, K_ref, rtol=0, atol=1e-12)
    assert np.allclose(V, (u @ Wv).reshape(T, H, dh), rtol=0, atol=1e-12)


def test_one_hot_rows_read_out_the_map():
    # x = e_j gives h = W[j, :] + b; with gamma = 1, eps = 0, W_V = I, V = h / rms(h).
    rng = np.random.default_rng(2)
    d = 8
    W = rng.standard_normal((d, d))
    b = rng.standard_normal(d)
    for j in range(d):
        x = np.zeros((1, d))
        x[0, j] = 1.0
        _, V = oracle.fill_layer(x, W, b, np.ones(d), np.eye(d), np.eye(d), np.array([0.0]),
                                 2, 4, 0.0, 1e4)
        h = W[j] + b
        assert np.allclose(V.reshape(-1), h / np.sqrt(np.mean(h * h)), rtol=0, atol=1e-13)


def test_scale_invariance_pos_independence_and_range_split():
    rng = np.random.default_rng(3)
    d, H, dh, T = 24, 3, 8, 20
    X = rng.standard_normal((T, d))
    W, b, g, Wk, Wv = _rand_layer(rng, d, H * dh)
    (K, V), = oracle.fill(X, 0, T, 0, [(W, b, g, Wk, Wv)], H, dh, 0.0, 1e4)
    (K2, V2), = oracle.fill(X, 0, T, 0, [(3.5 * W, 3.5 * b, g, Wk, Wv)], H, dh, 0.0, 1e4)
    assert np.allclose(K, K2, atol=1e-12) and np.allclose(V, V2, atol=1e-12)
    # V does not depend on position; K at a shifted origin is K rotated further
    (K3, V3), = oracle.fill(X, 0, T, 1000, [(W, b, g, Wk, Wv)], H, dh, 0.0, 1e4)
    assert np.array_equal(V, V3)
    assert np.allclose(K3, oracle.rope_rotate(K, np.full(T, 1000.0), 1e4), atol=1e-12)
    # filling [0, 7) then [7, T) equals filling [0, T)
    (Ka, Va), = oracle.fill(X[:7], 0, 7, 0, [(W, b, g, Wk, Wv)], H, dh, 0.0, 1e4)
    (Kb, Vb), = oracle.fill(X[7:], 7, T, 0, [(W, b, g, Wk, Wv)], H, dh, 0.0, 1e4)
    assert np.allclose(np.concatenate([Ka, Kb]), K, atol=1e-13)
    assert np.allclose(np.concatenate([Va, Vb]), V, atol=1e-13)


def test_layer_subset_independence():
    rng = np.random.default_rng(4)
    d, H, dh, T = 16, 2, 4, 6
    X = rng.standard_normal((T, d))
    layers = [_rand_layer(rng, d, H * dh) for _ in range(3)]
    full = oracle.fill(X, 0, T, 0, layers, H, dh, 1e-6, 1e4)
    sub = oracle.fill(X, 0, T, 0, [layers[2], layers[0]], H, dh, 1e-6, 1e4)
    assert np.array_equal(sub[0][0], full[2][0]) and np.array_equal(sub[1][1], full[0][1])


def test_fill_rejects_row_count_mismatch():
    with pytest.raises(ValueError):
        oracle.fill(np.zeros((3, 4)), 0, 4, 0, [], 1, 4, 0.0, 1e4)


def test_per_head_key_norm_hand_worked_and_order():
    # one head of d_h = 4, identity map and projections, base 100, position 1, gamma_k =
    # [1, 2, 1, 1], eps_k = 0: x = [3, 4, 0, 0] has RMS 2.5 (the layer's RMSNorm with eps = 0
    # gives u = [1.2, 1.6, 0, 0], RMS 1); the key norm keeps it and scales dim 1 by 2:
    # [1.2, 3.2, 0, 0]; then the pairs (0, 2) and (1, 3) turn by 1 and 0.1 rad.  Rotating first
    # would scale the rotated dim 1 instead: 1.6 sin(0.1) in dim 3, not 3.2 sin(0.1).
    I = np.eye(4)
    K, V = oracle.fill_layer(np.array([[3.0, 4.0, 0.0, 0.0]]), I, np.zeros(4), np.ones(4), I, I,
                             np.array([1.0]), 1, 4, 0.0, 100.0, k_norm=np.array([1.0, 2.0, 1.0, 1.0]),
                             k_norm_eps=0.0)
    expect = [1.2 * math.cos(1.0), 3.2 * math.cos(0.1), 1.2 * math.sin(1.0), 3.2 * math.sin(0.1)]
    assert np.allclose(K[0, 0], expect, rtol=0, atol=1e-15)
    assert np.allclose(V[0, 0], [1.2, 1.6, 0.0, 0.0], rtol=0, atol=1e-15)


def test_per_head_key_norm_invariants():
    rng = np.random.default_rng(9)
    d, H, dh, n = 16, 2, 8, 5
    X = rng.standard_normal((n, d))
    W, Wk, Wv = rng.standard_normal((d, d)), rng.standard_normal((d, H * dh)), rng.standard_normal((d, H * dh))
    g, b = 1 + 0.1 * rng.standard_normal(d), rng.standard_normal(d)
    pos = np.arange(n, dtype=float) * 5
    K1, V1 = oracle.fill_layer(X, W, b, g, Wk, Wv, pos, H, dh, 1e-6, 1e4, k_norm=np.ones(dh), k_norm_eps=0.0)
    # unit gamma_k, no epsilon: every head of every key has RMS 1 (rotation keeps pair norms)
    assert np.allclose(np.sqrt(np.mean(K1 ** 2, axis=-1)), 1.0, rtol=0, atol=1e-12)
    # values untouched; keys invariant to a scale of W_K and to the head's own scale
    K0, V0 = oracle.fill_layer(X, W, b, g, Wk, Wv, pos, H, dh, 1e-6, 1e4)
    assert np.array_equal(V0, V1)
    K2, _ = oracle.fill_layer(X, W, b, g, 3.7 * Wk, Wv, pos, H, dh, 1e-6, 1e4, k_norm=np.ones(dh), k_norm_eps=0.0)
    assert np.allclose(K1, K2, rtol=0, atol=1e-12)
    # the normalised keys are the plain keys rescaled head by head before the rotation
    scale = 1.0 / np.sqrt(np.mean(oracle.rope_rotate(K0, -pos, 1e4) ** 2, axis=-1, keepdims=True))
    assert np.allclose(K1, K0 * scale, rtol=0, atol=1e-12)
