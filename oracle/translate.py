"""Token-wise linear KV-cache translators, fp64 (oracle; test infrastructure only).

KV-Lingo page, section 3.1 "Linear translator family":
  * each target layer l has its own token-wise linear maps, one for keys (T_K^l) and one for
    values (T_V^l), that read the caches of a set E_l of nu source layers;
  * head-wise translators are block-diagonal (target head h reads only source head h),
    head-mixing translators are unconstrained;
  * pre-norm storing: the maps act on the source's keys before any normalisation or
    rotation; the translated keys are normalised per head (for targets that normalise keys,
    section 2) and rotated by their token's position before they are stored.  Post-RoPE
    translators act on keys the source already rotated and store their output unrotated.
Section 3.1 "Source-layer selection": relative-depth match gives target layer l (1-based)
the band of nu consecutive source layers centred on c(l) = 1 + (l - 1)(N_src - 1)/(N_tgt - 1),
shifted at the boundaries so every band has nu layers.
Section 3.2, first training stage: the maps are fitted in closed form by minimising the
squared error, i.e. the ridge fit of ``oracle.ridge`` on (source rows, target rows).
Appendix "The R^2 assignment": each target layer reads the nu source layers whose
single-layer maps explain the largest fraction of its features (keys and values ranked apart).

Readings (where the page is silent):
  * nu source layers enter one map as the concatenation of their rows, so the map of a
    target layer is [nu * d_src, d_tgt] and the translation is the sum of the single-layer
    terms;
  * the band is the one whose middle is nearest c(l) among the bands that fit inside the
    source's layers; an exact tie goes to the deeper band; N_tgt = 1 reads c = 1;
  * the fitted maps carry the mean-centring intercept of the ridge fit (a zero intercept
    gives the purely linear map).

Convention: x-times-matrix, head-major columns (column g*d_h + j is head g, dim j).
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

from .fill import rmsnorm, rope_rotate
from .ridge import NotSPD, fit


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def relative_depth_centre(layer: int, n_src: int, n_tgt: int) -> Fraction:
    """c(l) for the 1-based target layer ``layer``, as an exact fraction."""
    if n_tgt == 1:
        return Fraction(1)
    return 1 + Fraction((layer - 1) * (n_src - 1), n_tgt - 1)


def relative_depth_sources(n_src: int, n_tgt: int, nu: int):
    """E_l for l = 1..n_tgt, as lists of 0-based source layer indices.

    Among the bands {s, ..., s + nu - 1} (1-based, 1 <= s <= n_src - nu + 1), take the one
    whose middle s + (nu - 1)/2 is nearest c(l); on an exact tie, the deeper one."""
    if not (1 <= nu <= n_src and n_tgt >= 1):
        raise ValueError("need 1 <= nu <= n_src and n_tgt >= 1")
    out = []
    for layer in range(1, n_tgt + 1):
        c = relative_depth_centre(layer, n_src, n_tgt)
        best = None
        for s in range(1, n_src - nu + 2):
            dist = abs(s + Fraction(nu - 1, 2) - c)
            if best is None or dist <= best[0]:
                best = (dist, s)
        s = best[1]
        out.append([s - 1 + j for j in range(nu)])
    return out


def headwise_dense(blocks) -> np.ndarray:
    """The dense [H*d_in, H*d_out] map of a head-wise translator given its per-head maps
    blocks [H, d_in, d_out] (block-diagonal: head g's inputs feed only head g's outputs)."""
    blocks = _f64(blocks)
    H, di, do = blocks.shape
    T = np.zeros((H * di, H * do))
    for g in range(H):
        T[g * di:(g + 1) * di, g * do:(g + 1) * do] = blocks[g]
    return T


def translate_layer(src_k, src_v, T_k, T_v, b_k, b_v, positions, n_kv_heads: int, head_dim: int,
                    base: float, k_norm=None, k_norm_eps: float = 1e-6):
    """Target K and V rows of one layer from its source rows.

    src_k, src_v [T, d_in]: the source keys (before rotation) and values of the nu source
    layers, concatenated along the row; T_k, T_v [d_in, H*d_h]; b_k, b_v [H*d_h] or None.
    k = src_k T_k + b_k, per-head RMS-normalised with gamma_k = ``k_norm`` when given, rotated
    by its position (not when ``base`` is None: post-RoPE translators act on keys the source
    already rotated and store their output as it is); v = src_v T_v + b_v.
    Returns (K, V), each [T, H, d_h] fp64."""
    src_k = _f64(src_k)
    src_v = _f64(src_v)
    n = src_k.shape[0]
    K = src_k @ _f64(T_k)
    V = src_v @ _f64(T_v)
    if b_k is not None:
        K = K + _f64(b_k)
    if b_v is not None:
        V = V + _f64(b_v)
    K = K.reshape(n, n_kv_heads, head_dim)
    V = V.reshape(n, n_kv_heads, head_dim)
    if k_norm is not None:
        K = rmsnorm(K, k_norm, k_norm_eps)
    if base is None:
        return K, V
    return rope_rotate(K, positions, base), V


def translate(t0: int, t1: int, pos0: int, layers, n_kv_heads: int, head_dim: int, base: float):
    """Translate token rows [t0, t1) of every listed target layer.

    ``layers`` is a sequence of (src_k, src_v, T_k, T_v, b_k, b_v) whose source rows are
    those of tokens t0..t1-1 (row i is token t0 + i).  Token t sits at RoPE position pos0 + t.
    Returns a list of (K, V) per layer, each [t1 - t0, H, d_h]."""
    positions = pos0 + np.arange(t0, t1, dtype=np.float64)
    out = []
    for sk, sv, Tk, Tv, bk, bv in layers:
        if _f64(sk).shape[0] != t1 - t0 or _f64(sv).shape[0] != t1 - t0:
            raise ValueError("source rows must be exactly the rows [t0, t1)")
        out.append(translate_layer(sk, sv, Tk, Tv, bk, bv, positions, n_kv_heads, head_dim, base))
    return out


def fit_translator(src_rows, tgt_rows, lam: float, mode: str = "absolute"):
    """First-stage closed-form translator: the ridge fit of the target rows [n, d_out] on the
    source rows [n, d_in] (mean-centred, intercept b).  Returns (T [d_in, d_out], b)."""
    return fit(src_rows, tgt_rows, lam, mode)


def fit_r2(src_rows, tgt_rows, lam: float, mode: str = "absolute") -> float:
    """R^2 of the closed-form map from one source layer's rows to one target layer's rows
    (KV-Lingo page, Appendix "The R^2 assignment": the fraction of the target layer's features
    explained by the map from source layer s alone, R^2 = 1 - r({s})).

    Written from its definition on the data: the ridge map with its intercept is fitted, the
    residual of every target feature is formed, and
        R^2 = 1 - ||Y - (X W + 1 b)||_F^2 / ||Y - 1 mean(Y)||_F^2."""
    X = _f64(src_rows)
    Y = _f64(tgt_rows)
    W, b = fit(X, Y, lam, mode)
    R = Y - (X @ W + b)
    Yc = Y - Y.mean(axis=0)
    return 1.0 - float(np.sum(R * R)) / float(np.sum(Yc * Yc))


def r2_assignment(r2, nu: int):
    """E_l for every target layer from a score matrix r2 [n_tgt][n_src]: the nu source layers
    with the highest R^2_l(s) (KV-Lingo page, Appendix "The R^2 assignment"), in ascending
    layer order.  Readings: equal scores go to the shallower source layer; NaN ranks last."""
    r2 = _f64(r2)
    n_tgt, n_src = r2.shape
    if not 1 <= nu <= n_src:
        raise ValueError("need 1 <= nu <= n_src")
    out = []
    for l in range(n_tgt):
        score = [(-np.inf if np.isnan(r2[l, s]) else r2[l, s]) for s in range(n_src)]
        order = sorted(range(n_src), key=lambda s: (-score[s], s))
        out.append(sorted(order[:nu]))
    return out


def greedy_sources(src_layers, tgt_rows, nu: int, lam: float, mode: str = "absolute"):
    """Greedy match (KV-Lingo page, section 3.1 "Source-layer selection"): forward selection
    over source layers on the residual of the ridge fit to the target layer.  Starting from
    no source, each step adds the source layer whose rows, taken together with those already
    chosen, leave the smallest residual, i.e. give the largest R^2 of the joint ridge fit
    (``fit_r2`` on the chosen layers' rows side by side, in ascending layer order).
    Readings: equal scores go to the shallower layer; a candidate set whose regularised Gram
    is not positive definite (lambda = 0 with a constant source layer, say) has no ridge map
    and ranks last.  src_layers: list of [n, d_src] arrays; tgt_rows: [n, d_out].  Returns
    the nu chosen layers, ascending."""
    n_src = len(src_layers)
    if not 1 <= nu <= n_src:
        raise ValueError("need 1 <= nu <= n_src")
    chosen = []
    for _ in range(nu):
        best = None
        for s in range(n_src):
            if s in chosen:
                continue
            cand = sorted(chosen + [s])
            try:
                score = fit_r2(np.hstack([_f64(src_layers[c]) for c in cand]), tgt_rows, lam, mode)
            except NotSPD:
                continue
            if best is None or score > best[0]:
                best = (score, s)
        if best is None:
            raise NotSPD(0)
        chosen.append(best[1])
    return sorted(chosen)
