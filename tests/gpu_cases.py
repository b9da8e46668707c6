"""Shared set-up for the GPU parity tests and the smoke check: draw a workload with the seeded
generators, run it through the C ABI, and compare with the oracle.  Not collected by pytest."""
from __future__ import annotations

import math
import sys
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np
import torch

import oracle
import synth

KV_TOL_BF16 = 2e-2   # max |K - K*| / RMS(K*) per layer and side, bf16 storage
KV_TOL_F32 = 1e-4    # fp32 storage: fp32 MFMA accumulation over d terms
W_TOL = 1e-3         # max |W - W*| / max |W*| per layer


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().double().numpy() if t.dtype == torch.bfloat16 else t.detach().cpu().double().numpy()


@dataclass
class FillCase:
    cfg: synth.Config
    t0: int
    t1: int
    pos0: int = 0
    chunk: Optional[int] = None
    n_layers: Optional[int] = None
    maps: Optional[str] = None
    sample: Optional[Sequence[int]] = None     # token indices to compare (None = all filled)
    gen_device: str = "cpu"                    # where inputs are drawn
    max_tokens: Optional[int] = None
    k_norm: bool = False                       # per-head key norm (gamma_k, eps 1e-6)
    composed: bool = False                     # rf_fill_compose + rf_fill_composed instead of rf_fill
    int8_maps: bool = False                    # weight-only int8 maps (rf_quantize_map)


def run_fill_case(case: FillCase, device="cuda"):
    """Fill [t0, t1) of every selected layer and compare against the oracle.

    Returns a dict of per-layer relative errors and sentinel status."""
    import linear_kv_cache_amd as rf
    from linear_kv_cache_amd.runner import ComposedFiller, Filler, alloc_cache, fill_weights, gather_rows

    cfg = case.cfg
    layers = cfg.filled_layers[: case.n_layers] if case.n_layers else cfg.filled_layers
    T = case.max_tokens or max(case.t1, cfg.prompt_tokens)
    gd = case.gen_device
    lws = [synth.layer_weights(cfg, l, device=gd, maps=case.maps) for l in layers]
    lws_dev = [synth.LayerWeights(*(x.to(device) for x in (w.W_map, w.b_map, w.gamma, w.W_k, w.W_v))) for w in lws]
    X = synth.hidden_states(cfg, case.t1 - case.t0, "prompt", device=gd).to(device)
    gks = [synth.key_norm_weights(cfg, l) for l in layers] if case.k_norm else None
    fw = fill_weights(cfg.d, cfg.n_kv_heads, cfg.head_dim, cfg.rms_eps, cfg.torch_dtype,
                      [w.W_map for w in lws_dev], [w.b_map for w in lws_dev], [w.gamma for w in lws_dev],
                      [w.W_k for w in lws_dev], [w.W_v for w in lws_dev],
                      k_norm=None if gks is None else [gk.to(device) for gk in gks], k_norm_eps=1e-6,
                      int8_maps=case.int8_maps)
    table = None
    if cfg.paged:
        table = synth.block_table(cfg, T, device=device)
    cache = alloc_cache(len(layers), cfg.n_kv_heads, cfg.head_dim, T, cfg.torch_dtype, device, paged=cfg.paged,
                        block_size=cfg.block_size, block_table=table,
                        n_blocks=(int(table.max()) + 1) if table is not None else None)
    chunk = case.chunk or (case.t1 - case.t0)
    if case.composed:
        filler = ComposedFiller(fw, cfg.rope_base, case.pos0 + T, chunk, device)
    else:
        filler = Filler(fw, cfg.rope_base, case.pos0 + T, chunk, device)
    for c0 in range(case.t0, case.t1, chunk):
        c1 = min(case.t1, c0 + chunk)
        filler.fill(X[c0 - case.t0: c1 - case.t0], c0, c1, case.pos0, cache)
    torch.cuda.synchronize()

    rows = np.arange(case.t0, case.t1) if case.sample is None else np.asarray(sorted(set(case.sample)))
    Xs = f64(X[torch.as_tensor(rows - case.t0, device=device)])
    out = {"k_err": [], "v_err": [], "sentinel_ok": True, "finite": True}
    tol = KV_TOL_F32 if cfg.dtype == "f32" else KV_TOL_BF16
    for li, w in enumerate(lws):
        # int8 maps: the oracle's own codes of the same fp32 map values, dequantised exactly
        W_ref = oracle.dequantize_rows(*oracle.quantize_rows(f64(w.W_map))) if case.int8_maps else f64(w.W_map)
        K_ref, V_ref = oracle.fill_layer(Xs, W_ref.T, f64(w.b_map), f64(w.gamma), f64(w.W_k).T,
                                         f64(w.W_v).T, case.pos0 + rows.astype(np.float64), cfg.n_kv_heads,
                                         cfg.head_dim, cfg.rms_eps, cfg.rope_base,
                                         None if gks is None else f64(gks[li]), 1e-6)
        Kall = gather_rows(cache, cache.k[li], 0, T)
        Vall = gather_rows(cache, cache.v[li], 0, T)
        ridx = torch.as_tensor(rows, device=device)
        K = f64(Kall[ridx])
        V = f64(Vall[ridx])
        ke = float(np.max(np.abs(K - K_ref)) / np.sqrt(np.mean(K_ref ** 2)))
        ve = float(np.max(np.abs(V - V_ref)) / np.sqrt(np.mean(V_ref ** 2)))
        out["k_err"].append(ke)
        out["v_err"].append(ve)
        # every filled row written and finite; everything else still the NaN sentinel
        filled = Kall[case.t0:case.t1]
        out["finite"] &= bool(torch.isfinite(filled.float()).all()) and bool(
            torch.isfinite(Vall[case.t0:case.t1].float()).all())
        for pool in (cache.k[li], cache.v[li]):
            vals = pool.view(-1, cfg.n_kv_heads * cfg.head_dim) if not cfg.paged else pool
            if not cfg.paged:
                outside = torch.ones(vals.shape[0], dtype=torch.bool, device=device)
                outside[case.t0:case.t1] = False
                out["sentinel_ok"] &= bool(torch.isnan(vals[outside].float()).all())
            else:
                blk = pool.view(-1, cfg.n_kv_heads, cfg.block_size, cfg.head_dim)
                unw = ~written_mask(cache, case.t0, case.t1, T)
                out["sentinel_ok"] &= bool(torch.isnan(blk.permute(0, 2, 1, 3)[unw].float()).all())
    out["tol"] = tol
    out["max_err"] = max(out["k_err"] + out["v_err"])
    return out


def written_mask(cache, t0, t1, T):
    """[n_blocks, block_size] mask of paged slots the fill of [t0, t1) writes."""
    bs = cache.desc.block_size
    n_blocks = cache.layout["n_blocks"]
    m = torch.zeros(n_blocks, bs, dtype=torch.bool, device=cache.k[0].device)
    t = torch.arange(t0, t1, device=m.device)
    phys = cache.block_table.long()[t // bs]
    m[phys, t % bs] = True
    return m


# ------------------------------------------------------------------------------------------
@dataclass
class FitCase:
    cfg: synth.Config
    rows: int
    chunks: Sequence[int]          # rows per accumulate call (sums to rows)
    lam: float
    mode: str = "absolute"
    n_targets: Optional[int] = None
    zero_column: Optional[int] = None


def draw_fit_data(case: FitCase, gen_device="cpu"):
    cfg = case.cfg
    nt = case.n_targets or cfg.n_targets
    X = synth.hidden_states(cfg, case.rows, "calib", device=gen_device)
    if case.zero_column is not None:
        X[:, case.zero_column] = 0
    Ys = [synth.late_layer_inputs(cfg, X, cfg.split + l) for l in range(nt)]
    return X, Ys


def run_fit_case(case: FitCase, device="cuda"):
    import linear_kv_cache_amd as rf
    from linear_kv_cache_amd.runner import GramState

    cfg = case.cfg
    X, Ys = draw_fit_data(case)
    nt = len(Ys)
    Xd = X.to(device)
    Yd = [Y.to(device) for Y in Ys]
    st = GramState(cfg.d, nt, cfg.torch_dtype, device)
    r0 = 0
    for c in case.chunks:
        st.accumulate(Xd[r0:r0 + c], [Y[r0:r0 + c] for Y in Yd])
        r0 += c
    assert r0 == case.rows
    mode = rf.RF_LAMBDA_ABSOLUTE if case.mode == "absolute" else rf.RF_LAMBDA_REL_MEAN_DIAG
    W, Wlp, b, info = st.solve(case.lam, mode, list(range(nt)))
    torch.cuda.synchronize()
    return dict(X=X, Ys=Ys, state=st, W=W, Wlp=Wlp, b=b, info=int(info.item()))


def fit_errors(res, case: FitCase):
    X, Ys = res["X"], res["Ys"]
    errs_w, errs_b = [], []
    Xn = f64(X)
    for l, Y in enumerate(Ys):
        W_ref, b_ref = oracle.fit(Xn, f64(Y), case.lam, case.mode)
        Wg = f64(res["W"][l]).T       # library stores out-feature major
        errs_w.append(float(np.max(np.abs(Wg - W_ref)) / np.max(np.abs(W_ref))))
        errs_b.append(float(np.max(np.abs(f64(res["b"][l]) - b_ref)) / max(np.max(np.abs(b_ref)), 1e-30)))
    return errs_w, errs_b


# ------------------------------------------------------------------------------------------
@dataclass
class TranslateCase:
    cfg: synth.TranslateConfig
    t0: int
    t1: int
    pos0: int = 0
    chunk: Optional[int] = None
    n_layers: Optional[int] = None
    sample: Optional[Sequence[int]] = None     # token indices to compare (None = all translated)
    gen_device: str = "cpu"
    k_norm: bool = False                       # the target's per-head key norm (eps 1e-6)
    rotate: bool = True                        # False: post-RoPE translators (no table)


def run_translate_case(case: TranslateCase, device="cuda"):
    """Translate [t0, t1) of the selected target layers through rf_translate and compare with
    the oracle on the same stored source rows and maps."""
    import linear_kv_cache_amd as rf
    from linear_kv_cache_amd.runner import Translator, alloc_cache, gather_rows, translate_weights

    cfg = case.cfg
    n_tgt = case.n_layers or cfg.n_tgt
    E = rf.rf_relative_depth_sources(cfg.n_src, cfg.n_tgt, cfg.nu)[:n_tgt]
    assert E == oracle.relative_depth_sources(cfg.n_src, cfg.n_tgt, cfg.nu)[:n_tgt]
    T = max(case.t1, cfg.tokens)
    gd = case.gen_device
    Ks, Vs = synth.source_cache(cfg, case.t1 - case.t0, device=gd, row_offset=case.t0)
    maps = [synth.translator_maps(cfg, l, device=gd) for l in range(n_tgt)]
    Kd, Vd = Ks.to(device), Vs.to(device)
    md = [tuple(None if x is None else x.to(device) for x in m) for m in maps]
    gks = [synth.key_norm_weights(cfg, l) for l in range(n_tgt)] if case.k_norm else None
    tw = translate_weights(cfg.d_in, cfg.n_kv_heads, cfg.head_dim, cfg.torch_dtype, [m[0] for m in md],
                           [m[1] for m in md], [m[2] for m in md] if cfg.bias else None,
                           [m[3] for m in md] if cfg.bias else None, headwise=cfg.maps == "headwise",
                           k_norm=None if gks is None else [gk.to(device) for gk in gks], k_norm_eps=1e-6)
    table = synth.translate_block_table(cfg, T, device=device) if cfg.paged else None
    cache = alloc_cache(n_tgt, cfg.n_kv_heads, cfg.head_dim, T, cfg.torch_dtype, device, paged=cfg.paged,
                        block_size=cfg.block_size, block_table=table,
                        n_blocks=(int(table.max()) + 1) if table is not None else None)
    base = cfg.rope_base if case.rotate else None
    tr = Translator(tw, base, case.pos0 + T, device)
    ld = cfg.n_src * cfg.d_src
    chunk = case.chunk or (case.t1 - case.t0)
    for c0 in range(case.t0, case.t1, chunk):
        c1 = min(case.t1, c0 + chunk)
        r0 = c0 - case.t0
        # a band of consecutive source layers is one row segment of the token-major source
        tr.translate([Kd[r0, e[0]] for e in E], [Vd[r0, e[0]] for e in E], ld, c0, c1, case.pos0, cache)
    torch.cuda.synchronize()

    rows = np.arange(case.t0, case.t1) if case.sample is None else np.asarray(sorted(set(case.sample)))
    ridx = torch.as_tensor(rows - case.t0)
    Kn, Vn = f64(Ks[ridx]), f64(Vs[ridx])
    out = {"k_err": [], "v_err": [], "sentinel_ok": True, "finite": True}
    tol = KV_TOL_F32 if cfg.dtype == "f32" else KV_TOL_BF16
    for li, (e, m) in enumerate(zip(E, maps)):
        sk = Kn[:, e[0]:e[0] + cfg.nu].reshape(len(rows), -1)
        sv = Vn[:, e[0]:e[0] + cfg.nu].reshape(len(rows), -1)
        K_ref, V_ref = oracle.translate_layer(sk, sv, f64(m[0]).T, f64(m[1]).T,
                                              None if m[2] is None else f64(m[2]),
                                              None if m[3] is None else f64(m[3]),
                                              case.pos0 + rows.astype(np.float64), cfg.n_kv_heads, cfg.head_dim,
                                              base, None if gks is None else f64(gks[li]), 1e-6)
        Kall = gather_rows(cache, cache.k[li], 0, T)
        Vall = gather_rows(cache, cache.v[li], 0, T)
        di = torch.as_tensor(rows, device=device)
        K, V = f64(Kall[di]), f64(Vall[di])
        out["k_err"].append(float(np.max(np.abs(K - K_ref)) / np.sqrt(np.mean(K_ref ** 2))))
        out["v_err"].append(float(np.max(np.abs(V - V_ref)) / np.sqrt(np.mean(V_ref ** 2))))
        out["finite"] &= bool(torch.isfinite(Kall[case.t0:case.t1].float()).all()) and bool(
            torch.isfinite(Vall[case.t0:case.t1].float()).all())
        for pool in (cache.k[li], cache.v[li]):
            if not cfg.paged:
                vals = pool.view(-1, cfg.kv_width)
                outside = torch.ones(vals.shape[0], dtype=torch.bool, device=device)
                outside[case.t0:case.t1] = False
                out["sentinel_ok"] &= bool(torch.isnan(vals[outside].float()).all())
            else:
                blk = pool.view(-1, cfg.n_kv_heads, cfg.block_size, cfg.head_dim)
                unw = ~written_mask(cache, case.t0, case.t1, T)
                out["sentinel_ok"] &= bool(torch.isnan(blk.permute(0, 2, 1, 3)[unw].float()).all())
    out["tol"] = tol
    out["max_err"] = max(out["k_err"] + out["v_err"])
    return out
