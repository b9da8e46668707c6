"""The pins are sharp: a plausible mistake planted in (a copy of) the oracle fails them.

Mistakes are planted on the CPU only, by wrapping the oracle's functions."""
import math

import numpy as np

import oracle


def _planted_recovers(fit):
    rng = np.random.default_rng(3)
    X = rng.standard_normal((200, 12)) + 0.7
    A = rng.standard_normal((12, 5))
    c = rng.standard_normal(5)
    W, b = fit(X, X @ A + c, 1e-9)
    return np.allclose(W, A, atol=1e-6) and np.allclose(b, c, atol=1e-6)


def test_fit_pins_catch_mistakes():
    assert _planted_recovers(oracle.fit)

    def no_intercept(X, Y, lam):
        W, _ = oracle.fit(X, Y, lam)
        return W, np.zeros(W.shape[1])

    def uncentred(X, Y, lam):
        X = np.asarray(X, float)
        Y = np.asarray(Y, float)
        W = np.linalg.solve(X.T @ X + lam * np.eye(X.shape[1]), X.T @ Y)
        return W, Y.mean(0) - X.mean(0) @ W

    def transposed(X, Y, lam):
        W, b = oracle.fit(X, Y, lam)
        return W.T[:W.shape[0], :W.shape[1]] if W.shape[0] == W.shape[1] else W[::-1], b

    for bad in (no_intercept, uncentred, transposed):
        assert not _planted_recovers(bad)


def _hand_example(rope):
    u = np.array([[[1.2, 1.6, 0.0, 0.0]]])
    k = rope(u, np.array([1.0]), 100.0)[0, 0]
    want = [1.2 * math.cos(1.0), 1.6 * math.cos(0.1), 1.2 * math.sin(1.0), 1.6 * math.sin(0.1)]
    return np.allclose(k, want, atol=1e-12)


def test_rope_pins_catch_mistakes():
    assert _hand_example(oracle.rope_rotate)

    def wrong_sign(k, pos, base):
        return oracle.rope_rotate(k, -np.asarray(pos), base)

    def interleaved_pairs(k, pos, base):
        k = np.asarray(k, float)
        perm = np.arange(k.shape[-1]).reshape(2, -1).T.reshape(-1)  # (0,h,1,h+1,...)
        r = oracle.rope_rotate(k[..., perm], pos, base)
        out = np.empty_like(r)
        out[..., perm] = r
        return out

    def wrong_frequency(k, pos, base):
        return oracle.rope_rotate(k, pos, base ** 2)

    for bad in (wrong_sign, interleaved_pairs, wrong_frequency):
        assert not _hand_example(bad)


def _translator_pins_hold(tl):
    # identity map = rotation of the source (complex route); head-wise = head by head
    rng = np.random.default_rng(8)
    H, dh, n = 2, 8, 6
    sk, sv = rng.standard_normal((n, H * dh)), rng.standard_normal((n, H * dh))
    pos = 1.0 + np.arange(n) * 7
    half = dh // 2
    theta = np.array([1e4 ** (-(2.0 * i) / dh) for i in range(half)])
    ok = True
    K, V = tl(sk, sv, np.eye(H * dh), np.eye(H * dh), None, None, pos, H, dh, 1e4)
    z = (sk.reshape(n, H, dh)[..., :half] + 1j * sk.reshape(n, H, dh)[..., half:]) * np.exp(
        1j * pos[:, None, None] * theta)
    ok &= np.allclose(K, np.concatenate([z.real, z.imag], -1), atol=1e-12)
    ok &= np.allclose(V, sv.reshape(n, H, dh), atol=1e-12)
    blocks = rng.standard_normal((H, dh, dh))
    T = oracle.headwise_dense(blocks)
    _, V2 = tl(sk, sv, T, T, None, None, np.zeros(n), H, dh, 1e4)
    for g in range(H):
        ok &= np.allclose(V2[:, g], sv[:, g * dh:(g + 1) * dh] @ blocks[g], atol=1e-12)
    Tm = rng.standard_normal((H * dh, H * dh))
    K3, _ = tl(sk, sv, Tm, Tm, None, None, pos, H, dh, 1e4)
    ok &= np.allclose(K3, oracle.rope_rotate((sk @ Tm).reshape(n, H, dh), pos, 1e4), atol=1e-12)
    return bool(ok)


def test_translator_pins_catch_mistakes():
    assert _translator_pins_hold(oracle.translate_layer)

    def transposed_map(sk, sv, Tk, Tv, bk, bv, pos, H, dh, base):
        return oracle.translate_layer(sk, sv, np.asarray(Tk).T, np.asarray(Tv).T, bk, bv, pos, H, dh, base)

    def rotates_values_too(sk, sv, Tk, Tv, bk, bv, pos, H, dh, base):
        K, V = oracle.translate_layer(sk, sv, Tk, Tv, bk, bv, pos, H, dh, base)
        return K, oracle.rope_rotate(V, pos, base)

    def rotates_before_the_map(sk, sv, Tk, Tv, bk, bv, pos, H, dh, base):
        n = np.asarray(sk).shape[0]
        rk = oracle.rope_rotate(np.asarray(sk, float).reshape(n, H, dh), pos, base).reshape(n, -1)
        _, V = oracle.translate_layer(sk, sv, Tk, Tv, bk, bv, pos, H, dh, base)
        return (rk @ np.asarray(Tk, float)).reshape(n, H, dh), V

    for bad in (transposed_map, rotates_values_too, rotates_before_the_map):
        assert not _translator_pins_hold(bad)


def test_relative_depth_pins_catch_mistakes():
    def holds(sel):
        return (sel(28, 36, 3)[17] == [12, 13, 14] and sel(28, 36, 3)[35] == [25, 26, 27]
                and sel(3, 5, 1)[1] == [1] and sel(7, 7, 1) == [[l] for l in range(7)])

    assert holds(oracle.relative_depth_sources)

    def ties_to_shallower(n_src, n_tgt, nu):
        from fractions import Fraction
        out = []
        for l in range(1, n_tgt + 1):
            c = oracle.relative_depth_centre(l, n_src, n_tgt)
            s = min(range(1, n_src - nu + 2), key=lambda s: abs(s + Fraction(nu - 1, 2) - c))
            out.append([s - 1 + j for j in range(nu)])
        return out

    def unshifted_at_ends(n_src, n_tgt, nu):
        out = []
        for l in range(1, n_tgt + 1):
            c = oracle.relative_depth_centre(l, n_src, n_tgt)
            s = int(np.floor(c - (nu - 1) / 2 + 0.5))
            out.append([s - 1 + j for j in range(nu)])
        return out

    def truncates_centre(n_src, n_tgt, nu):
        out = []
        for l in range(1, n_tgt + 1):
            c = 1 + (l - 1) * (n_src - 1) // max(1, n_tgt - 1)
            s = min(max(1, c - (nu - 1) // 2), n_src - nu + 1)
            out.append([s - 1 + j for j in range(nu)])
        return out

    for bad in (ties_to_shallower, unshifted_at_ends, truncates_centre):
        assert not holds(bad)


def _gdn_pins_hold(gdn):
    # the hand-worked token and the exact write of the delta rule
    ok = np.allclose(gdn(np.array([[[0.6, 0.8]]]), np.array([[[3.0]]]), np.log([[0.5]]), np.array([[0.5]]),
                         S0=np.array([[[1.0, 2.0]]])), [[[1.07, 1.76]]], atol=1e-12)
    rng = np.random.default_rng(9)
    S0 = rng.standard_normal((1, 3, 4))
    k = np.array([0.5, 0.5, 0.5, 0.5])
    v = rng.standard_normal(3)
    S = gdn(k[None, None, :], v[None, None, :], np.log([[0.6]]), np.ones((1, 1)), S0=S0)
    return ok and np.allclose(S[0] @ k, v, atol=1e-12)


def test_gdn_pins_catch_mistakes():
    assert _gdn_pins_hold(oracle.gdn_state)

    def decay_after_write(K, V, g, beta, S0=None, normalise_k=False):
        S = np.array(S0, float)
        for t in range(K.shape[0]):
            for h in range(K.shape[1]):
                k, a, b = K[t, h], np.exp(g[t, h]), beta[t, h]
                S[h] = a * (S[h] - b * np.outer(S[h] @ k, k) + b * np.outer(V[t, h], k))
        return S

    def erase_without_beta(K, V, g, beta, S0=None, normalise_k=False):
        S = np.array(S0, float)
        for t in range(K.shape[0]):
            for h in range(K.shape[1]):
                k, a, b = K[t, h], np.exp(g[t, h]), beta[t, h]
                S[h] = a * (S[h] - np.outer(S[h] @ k, k)) + b * np.outer(V[t, h], k)
        return S

    for bad in (decay_after_write, erase_without_beta):
        assert not _gdn_pins_hold(bad)


def _quant_pins_hold(qr):
    # the hand-worked grid and tie rows of tests/test_oracle_quant.py, and the half-step bound
    s0 = np.float32(2.0 ** -7)
    grid = s0 * np.array([[127, -64, 3, 0, -127, 1]], dtype=np.float32)
    ties = s0 * np.array([[127, 2.5, 3.5, -2.5, -0.5, 0.5, 1.5, -126.5]], dtype=np.float32)
    neg = np.zeros((1, 5), dtype=np.float32)
    neg[0, 3] = -0.75
    q1, s1 = qr(grid)
    q2, _ = qr(ties)
    q3, _ = qr(neg)
    ok = (np.array_equal(q1, [[127, -64, 3, 0, -127, 1]]) and float(s1[0]) == float(s0)
          and np.array_equal(q2, [[127, 2, 4, -2, 0, 0, 2, -126]]) and np.array_equal(q3, [[0, 0, 0, -127, 0]]))
    rng = np.random.default_rng(11)
    W = rng.standard_normal((8, 64)).astype(np.float32)
    q, s = qr(W)
    err = np.abs(np.asarray(s, np.float64)[:, None] * np.asarray(q, np.float64) - W)
    return bool(ok and np.all(err <= np.asarray(s, np.float64)[:, None] * (0.5 + 1e-5)))


def test_quantiser_pins_catch_mistakes():
    assert _quant_pins_hold(oracle.quantize_rows)

    def truncates(W):
        W = np.asarray(W, np.float32)
        s = (np.max(np.abs(W), axis=1) / np.float32(127)).astype(np.float32)
        return np.trunc(W / np.where(s > 0, s, 1)[:, None]).astype(np.int8), s

    def ties_away(W):
        W = np.asarray(W, np.float32)
        s = (np.max(np.abs(W), axis=1) / np.float32(127)).astype(np.float32)
        x = W / np.where(s > 0, s, 1)[:, None]
        return (np.sign(x) * np.floor(np.abs(x) + 0.5)).astype(np.int8), s

    def scale_by_128(W):
        W = np.asarray(W, np.float32)
        s = (np.max(np.abs(W), axis=1) / np.float32(128)).astype(np.float32)
        return np.clip(np.rint(W / np.where(s > 0, s, 1)[:, None]), -127, 127).astype(np.int8), s

    def signed_maximum(W):
        W = np.asarray(W, np.float32)
        s = np.abs(np.max(W, axis=1) / np.float32(127)).astype(np.float32)
        return np.clip(np.rint(W / np.where(s > 0, s, 1)[:, None]), -127, 127).astype(np.int8), s

    for bad in (truncates, ties_away, scale_by_128, signed_maximum):
        assert not _quant_pins_hold(bad), bad.__name__
