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
