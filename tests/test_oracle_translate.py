"""Pins of the oracle's KV-cache translators (KV-Lingo page, sections 3.1-3.2) against closed
forms, hand-worked cases and invariants (CPU only)."""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle


def _rope_complex(k, positions, base):
    # independent route: pair (i, i+h) as the complex number a + i c, times e^{i pos theta}
    half = k.shape[-1] // 2
    theta = np.array([base ** (-(2.0 * i) / k.shape[-1]) for i in range(half)])
    z = (k[..., :half] + 1j * k[..., half:]) * np.exp(1j * positions[:, None, None] * theta)
    return np.concatenate([z.real, z.imag], axis=-1)


# ---- relative-depth source selection ---------------------------------------------------------

def test_relative_depth_hand_worked():
    # N_src = 28, N_tgt = 36, nu = 3: c(l) = 1 + 27 (l - 1) / 35
    #   l = 1  -> c = 1;        the centred band {0, 1, 2} (1-based) is shifted to {1, 2, 3}
    #   l = 18 -> c = 494/35 = 14.11; band centred on 14: {13, 14, 15}
    #   l = 36 -> c = 28;       band {27, 28, 29} shifted to {26, 27, 28}
    E = oracle.relative_depth_sources(28, 36, 3)
    assert oracle.relative_depth_centre(18, 28, 36) == Fraction(494, 35)
    assert E[0] == [0, 1, 2]
    assert E[17] == [12, 13, 14]
    assert E[35] == [25, 26, 27]
    # a tie: N_src = 3, N_tgt = 5 gives c(2) = 3/2, half-way between layers 1 and 2; nu = 1
    # takes the deeper one; nu = 2 is centred exactly on it
    assert oracle.relative_depth_centre(2, 3, 5) == Fraction(3, 2)
    assert oracle.relative_depth_sources(3, 5, 1)[1] == [1]
    assert oracle.relative_depth_sources(3, 5, 2)[1] == [0, 1]


def test_relative_depth_shape_preserving_and_ends():
    # the page: a shape-preserving pair reads its counterpart, E_l = {l}
    for n in (1, 2, 7, 36):
        assert oracle.relative_depth_sources(n, n, 1) == [[l] for l in range(n)]
    for n_src, n_tgt in [(28, 36), (36, 28), (64, 32), (5, 17), (2, 2)]:
        c_first = oracle.relative_depth_centre(1, n_src, n_tgt)
        c_last = oracle.relative_depth_centre(n_tgt, n_src, n_tgt)
        assert c_first == 1 and c_last == n_src
        for nu in range(1, n_src + 1):
            E = oracle.relative_depth_sources(n_src, n_tgt, nu)
            assert len(E) == n_tgt
            assert E[0] == list(range(nu))
            assert E[-1] == list(range(n_src - nu, n_src))
            starts = [e[0] for e in E]
            assert starts == sorted(starts)                     # deeper targets read deeper
            for e in E:
                assert e == list(range(e[0], e[0] + nu)) and 0 <= e[0] and e[-1] < n_src


def test_relative_depth_band_is_nearest_to_centre():
    # brute force: no other band of nu layers inside the source has its middle closer to c
    for n_src, n_tgt, nu in [(28, 36, 3), (36, 28, 4), (9, 9, 2), (12, 40, 5)]:
        E = oracle.relative_depth_sources(n_src, n_tgt, nu)
        for l, e in enumerate(E, start=1):
            c = oracle.relative_depth_centre(l, n_src, n_tgt)
            mid = e[0] + 1 + Fraction(nu - 1, 2)
            for s in range(1, n_src - nu + 2):
                assert abs(mid - c) <= abs(s + Fraction(nu - 1, 2) - c)


def test_relative_depth_rejects_bad_sizes():
    with pytest.raises(ValueError):
        oracle.relative_depth_sources(4, 4, 5)
    with pytest.raises(ValueError):
        oracle.relative_depth_sources(4, 0, 1)


# ---- translation --------------------------------------------------------------------------

def test_identity_translator_is_rope_of_the_source():
    # T = I, no intercept: the target keys are the source keys rotated, values unchanged;
    # the rotation is checked by the complex-multiplication route
    rng = np.random.default_rng(1)
    H, dh, n = 3, 8, 11
    sk = rng.standard_normal((n, H * dh))
    sv = rng.standard_normal((n, H * dh))
    pos = 5 + np.arange(n, dtype=float) * 1000
    K, V = oracle.translate_layer(sk, sv, np.eye(H * dh), np.eye(H * dh), None, None, pos, H, dh, 1e4)
    assert np.allclose(K, _rope_complex(sk.reshape(n, H, dh), pos, 1e4), rtol=0, atol=1e-12)
    assert np.array_equal(V, sv.reshape(n, H, dh))


def test_hand_worked_one_hot_translation():
    # one head of d_h = 2, base 100 (theta_0 = 1): source key e_1 picks row 1 of T_k,
    # [0.5, -2] + b [1, 1] = [1.5, -1]; at position 2 it turns by 2 rad
    T = np.array([[9.0, 9.0], [0.5, -2.0]])
    K, V = oracle.translate_layer([[0.0, 1.0]], [[0.0, 1.0]], T, T, [1.0, 1.0], [0.0, 0.0],
                                  np.array([2.0]), 1, 2, 100.0)
    a, c = 1.5, -1.0
    assert np.allclose(K[0, 0], [a * math.cos(2) - c * math.sin(2), c * math.cos(2) + a * math.sin(2)],
                       rtol=0, atol=1e-15)
    assert np.allclose(V[0, 0], [0.5, -2.0], rtol=0, atol=1e-15)


def test_headwise_translator_acts_head_by_head():
    # block-diagonal map = each target head g computed from source head g alone
    rng = np.random.default_rng(2)
    H, dh, n = 4, 6, 9
    blocks_k = rng.standard_normal((H, dh, dh))
    blocks_v = rng.standard_normal((H, dh, dh))
    sk = rng.standard_normal((n, H * dh))
    sv = rng.standard_normal((n, H * dh))
    pos = np.arange(n, dtype=float) + 17
    K, V = oracle.translate_layer(sk, sv, oracle.headwise_dense(blocks_k), oracle.headwise_dense(blocks_v),
                                  None, None, pos, H, dh, 5e5)
    for g in range(H):
        kg = sk[:, g * dh:(g + 1) * dh] @ blocks_k[g]
        vg = sv[:, g * dh:(g + 1) * dh] @ blocks_v[g]
        assert np.allclose(K[:, g], _rope_complex(kg[:, None, :], pos, 5e5)[:, 0], rtol=0, atol=1e-12)
        assert np.allclose(V[:, g], vg, rtol=0, atol=1e-12)
    # and the dense matrix has zeros off the diagonal blocks
    T = oracle.headwise_dense(blocks_k)
    assert np.count_nonzero(T) == H * dh * dh


def test_multi_source_is_the_sum_of_single_sources():
    # nu = 2: [k1 | k2] [T1; T2] + b = (k1 T1) + (k2 T2) + b, and RoPE is linear
    rng = np.random.default_rng(3)
    H, dh, n = 2, 8, 7
    k1, k2, v1, v2 = (rng.standard_normal((n, H * dh)) for _ in range(4))
    T1, T2, U1, U2 = (rng.standard_normal((H * dh, H * dh)) for _ in range(4))
    b = rng.standard_normal(H * dh)
    pos = np.arange(n, dtype=float) * 3
    K, V = oracle.translate_layer(np.hstack([k1, k2]), np.hstack([v1, v2]), np.vstack([T1, T2]),
                                  np.vstack([U1, U2]), b, b, pos, H, dh, 1e4)
    Ka, Va = oracle.translate_layer(k1, v1, T1, U1, b, b, pos, H, dh, 1e4)
    Kb, Vb = oracle.translate_layer(k2, v2, T2, U2, None, None, pos, H, dh, 1e4)
    assert np.allclose(K, Ka + Kb, rtol=0, atol=1e-12)
    assert np.allclose(V, Va + Vb, rtol=0, atol=1e-12)


def test_positions_turn_keys_only():
    rng = np.random.default_rng(4)
    H, dh, n = 2, 8, 5
    sk, sv = rng.standard_normal((n, H * dh)), rng.standard_normal((n, H * dh))
    Tk, Tv = rng.standard_normal((H * dh, H * dh)), rng.standard_normal((H * dh, H * dh))
    K0, V0 = oracle.translate_layer(sk, sv, Tk, Tv, None, None, np.zeros(n), H, dh, 1e4)
    assert np.allclose(K0.reshape(n, -1), sk @ Tk, rtol=0, atol=1e-12)   # position 0: no turn
    pos = np.array([1.0, 10, 100, 1000, 100000])
    K1, V1 = oracle.translate_layer(sk, sv, Tk, Tv, None, None, pos, H, dh, 1e4)
    assert np.array_equal(V0, V1)
    assert np.allclose(K1, oracle.rope_rotate(K0, pos, 1e4), rtol=0, atol=1e-12)


def test_translate_range_and_layers():
    rng = np.random.default_rng(5)
    H, dh = 2, 4
    mk = lambda: (rng.standard_normal((6, H * dh)), rng.standard_normal((6, H * dh)),
                  rng.standard_normal((H * dh, H * dh)), rng.standard_normal((H * dh, H * dh)), None, None)
    layers = [mk(), mk()]
    out = oracle.translate(10, 16, 3, layers, H, dh, 1e4)
    pos = 3 + np.arange(10, 16, dtype=float)
    for (K, V), lw in zip(out, layers):
        K1, V1 = oracle.translate_layer(*lw, pos, H, dh, 1e4)
        assert np.array_equal(K, K1) and np.array_equal(V, V1)
    with pytest.raises(ValueError):
        oracle.translate(10, 15, 0, layers, H, dh, 1e4)


def test_fit_translator_recovers_a_planted_map():
    # target rows exactly an affine map of the source rows: the closed-form first stage
    # recovers it (lambda -> 0), and translating with it reproduces the target cache
    rng = np.random.default_rng(6)
    H, dh, n = 2, 8, 300
    src = rng.standard_normal((n, H * dh)) * 2 + 0.3
    T = rng.standard_normal((H * dh, H * dh)) / 4
    c = rng.standard_normal(H * dh)
    tgt = src @ T + c
    Tf, bf = oracle.fit_translator(src, tgt, 1e-10)
    assert np.allclose(Tf, T, rtol=0, atol=1e-8) and np.allclose(bf, c, rtol=0, atol=1e-8)
    # head-wise planted map: the fit of each head's columns on its own source head recovers
    # the blocks
    blocks = rng.standard_normal((H, dh, dh))
    tgt_h = src @ oracle.headwise_dense(blocks)
    for g in range(H):
        Tg, bg = oracle.fit_translator(src[:, g * dh:(g + 1) * dh], tgt_h[:, g * dh:(g + 1) * dh], 1e-10)
        assert np.allclose(Tg, blocks[g], rtol=0, atol=1e-8) and np.allclose(bg, 0, atol=1e-8)


# ---- R^2 of single-layer maps and the R^2 assignment ----------------------------------------

def test_r2_one_feature_is_squared_correlation():
    # textbook identity: for one source feature and one target feature, the least-squares fit
    # with an intercept explains corr(x, y)^2 of the target's variance
    rng = np.random.default_rng(10)
    x = rng.standard_normal((500, 1))
    y = 0.7 * x + rng.standard_normal((500, 1))
    rho = np.corrcoef(x[:, 0], y[:, 0])[0, 1]
    assert abs(oracle.fit_r2(x, y, 0.0) - rho ** 2) <= 1e-12


def test_r2_limits_and_monotone_in_lambda():
    rng = np.random.default_rng(11)
    X = rng.standard_normal((400, 12)) + 1.5
    A = rng.standard_normal((12, 6))
    assert abs(oracle.fit_r2(X, X @ A + 3.0, 1e-10) - 1.0) <= 1e-10       # exact affine map
    E = rng.standard_normal((400, 6))
    vals = [oracle.fit_r2(X, X @ A + E, lam) for lam in (0.0, 1.0, 100.0, 1e4, 1e8)]
    assert all(0.0 <= v <= 1.0 for v in vals)
    assert all(a > b for a, b in zip(vals, vals[1:]))                     # more shrinkage, less fit
    assert vals[-1] < 1e-3                                                # lambda -> inf: W -> 0
    # a target independent of the source: R^2 near 0 (expected d / n for least squares)
    r0 = oracle.fit_r2(X, rng.standard_normal((400, 6)), 0.0)
    assert 0.0 <= r0 < 0.1


def test_r2_from_the_sums_equals_the_data_route():
    # the scores can be read off the accumulated sums (the page: no extra pass over the data):
    # SSE = SST - sum(W * B) - lambda ||W||^2 with B the centred cross moments
    rng = np.random.default_rng(12)
    X = rng.standard_normal((300, 10)) * np.linspace(0.5, 2, 10) + 0.3
    Y = X @ rng.standard_normal((10, 7)) + 0.5 * rng.standard_normal((300, 7)) - 1.0
    lam = 5.0
    S_xx, S_xy, s_x, s_y, n = oracle.gram_sums(X, [Y])
    (W, b), = oracle.fit_from_sums(S_xx, S_xy, s_x, s_y, n, lam)
    B = S_xy[0] - np.outer(s_x, s_y[0]) / n
    SST = float(np.sum(Y * Y) - np.sum(s_y[0] ** 2) / n)
    r2_sums = (float(np.sum(W * B)) + lam * float(np.sum(W * W))) / SST
    assert abs(r2_sums - oracle.fit_r2(X, Y, lam)) <= 1e-12


def test_r2_assignment_hand_worked():
    r2 = np.array([[0.1, 0.9, 0.5, 0.9],     # tie 0.9 at sources 1 and 3: both kept for nu = 2
                   [0.8, 0.2, 0.8, 0.3],     # tie at 0 and 2 for nu = 1: the shallower, 0
                   [0.0, 0.0, 0.0, 0.0]])
    assert oracle.r2_assignment(r2, 1) == [[1], [0], [0]]
    assert oracle.r2_assignment(r2, 2) == [[1, 3], [0, 2], [0, 1]]
    assert oracle.r2_assignment(r2, 4) == [[0, 1, 2, 3]] * 3
    with pytest.raises(ValueError):
        oracle.r2_assignment(r2, 5)


def test_translator_key_norm_before_rotation():
    # pre-norm storing: map, then the target's per-head key norm, then RoPE (KV-Lingo section 3.1)
    rng = np.random.default_rng(13)
    H, dh, n = 2, 8, 6
    sk, sv = rng.standard_normal((n, H * dh)), rng.standard_normal((n, H * dh))
    Tk, Tv = rng.standard_normal((H * dh, H * dh)), rng.standard_normal((H * dh, H * dh))
    gk = 1 + 0.2 * rng.standard_normal(dh)
    pos = 3.0 + np.arange(n)
    K, V = oracle.translate_layer(sk, sv, Tk, Tv, None, None, pos, H, dh, 1e4, k_norm=gk, k_norm_eps=1e-6)
    k = (sk @ Tk).reshape(n, H, dh)
    kn = k / np.sqrt(np.mean(k * k, axis=-1, keepdims=True) + 1e-6) * gk
    assert np.allclose(K, _rope_complex(kn, pos, 1e4), rtol=0, atol=1e-12)
    assert np.allclose(V, (sv @ Tv).reshape(n, H, dh), rtol=0, atol=1e-12)


def test_post_rope_translators_store_unrotated():
    # post-RoPE capture: the maps act on keys the source already rotated, nothing is turned
    # after the map; rotation commutes with a map that acts on each rotation pair as a complex
    # scalar, so rotating then translating equals translating then rotating for such maps
    rng = np.random.default_rng(14)
    H, dh, n = 2, 8, 5
    sk, sv = rng.standard_normal((n, H * dh)), rng.standard_normal((n, H * dh))
    pos = 2.0 + np.arange(n) * 11
    K, V = oracle.translate_layer(sk, sv, np.eye(H * dh), np.eye(H * dh), None, None, pos, H, dh, None)
    assert np.array_equal(K, sk.reshape(n, H, dh)) and np.array_equal(V, sv.reshape(n, H, dh))
    # per pair: (a, c) -> (alpha a - beta c, beta a + alpha c) is multiplication by alpha + i beta
    half = dh // 2
    alpha, beta = rng.standard_normal(half), rng.standard_normal(half)
    blk = np.zeros((dh, dh))
    for i in range(half):
        blk[i, i], blk[i + half, i] = alpha[i], -beta[i]
        blk[i, i + half], blk[i + half, i + half] = beta[i], alpha[i]
    T = oracle.headwise_dense(np.stack([blk] * H))
    rotated = oracle.rope_rotate(sk.reshape(n, H, dh), pos, 1e4).reshape(n, -1)
    K_post, _ = oracle.translate_layer(rotated, sv, T, T, None, None, pos, H, dh, None)
    K_pre, _ = oracle.translate_layer(sk, sv, T, T, None, None, pos, H, dh, 1e4)
    assert np.allclose(K_post, K_pre, rtol=0, atol=1e-12)


def test_greedy_match_accounts_for_redundancy():
    # The page contrasts the two data-driven assignments: the R^2 assignment keeps two source
    # layers that explain the same part of the target, greedy match does not.  Sources 0 and 1
    # carry the same signal (1 is 0 plus a little noise), source 2 carries a weaker,
    # independent one, source 3 nothing; the target is their sum plus noise.
    rng = np.random.default_rng(15)
    n, d = 600, 6
    a, b = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    src = [a, a + 0.05 * rng.standard_normal((n, d)), b, rng.standard_normal((n, d))]
    tgt = a @ rng.standard_normal((d, 4)) + 0.5 * b @ rng.standard_normal((d, 4)) + 0.1 * rng.standard_normal((n, 4))
    r2 = np.array([[oracle.fit_r2(s, tgt, 1e-3) for s in src]])
    assert oracle.r2_assignment(r2, 2) == [[0, 1]]              # both copies of the same signal
    assert oracle.greedy_sources(src, tgt, 2, 1e-3) == [0, 2]   # the copy adds nothing new
    # one source: greedy and the R^2 assignment agree (the single best fit)
    assert oracle.greedy_sources(src, tgt, 1, 1e-3) == oracle.r2_assignment(r2, 1)[0]
    # all sources: everything
    assert oracle.greedy_sources(src, tgt, 4, 1e-3) == [0, 1, 2, 3]


def test_greedy_match_skips_sets_without_a_ridge_map():
    # lambda = 0 and a source layer of constant rows: every candidate set holding it has a
    # singular Gram (a zero row and column after centring), so no ridge map exists and the set
    # ranks last; the other sources are still chosen in their order of merit, and asking for
    # every source leaves no fittable set at the last step
    rng = np.random.default_rng(16)
    n, d = 400, 5
    a, b = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    src = [np.full((n, d), 0.75), a, b]
    tgt = a @ rng.standard_normal((d, 3)) + 0.3 * b @ rng.standard_normal((d, 3)) + 0.05 * rng.standard_normal((n, 3))
    with pytest.raises(oracle.NotSPD):
        oracle.fit_r2(src[0], tgt, 0.0)
    assert oracle.greedy_sources(src, tgt, 1, 0.0) == [1]
    assert oracle.greedy_sources(src, tgt, 2, 0.0) == [1, 2]
    with pytest.raises(oracle.NotSPD):
        oracle.greedy_sources(src, tgt, 3, 0.0)
    # with a ridge the constant layer is fittable again (and explains nothing)
    assert oracle.greedy_sources(src, tgt, 3, 1e-3) == [0, 1, 2]
