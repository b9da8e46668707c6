"""Parity at the workloads' full sizes, in the launch configuration the benchmark uses.

The fill is checked on sampled token rows (every chunk, tile and block boundary plus seeded
random rows) across all filled layers, with every unfilled row checked against its sentinel.
The fit is checked on sampled Gram entries and sampled output columns of every map: column
j of W depends only on column j of Y, so the oracle solves those columns exactly from the
full calibration set."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_cases import W_TOL, FillCase, f64, log, run_fill_case

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _boundary_sample(t0, t1, chunk, seed, n_random=24, block=16, tile=256):
    rng = np.random.default_rng(seed)
    s = {t0, t0 + 1, t1 - 1, t1 - 2}
    for c in range(t0, t1, chunk):
        s.update({c, c - 1, c + chunk - 1})
    for b in range(t0 - t0 % tile, t1, tile):
        s.update({b, b - 1})
    for b in range(t0 - t0 % block + block, min(t1, t0 + 8 * block), block):
        s.update({b - 1, b})
    s.update(rng.integers(t0, t1, n_random).tolist())
    return sorted(x for x in s if t0 <= x < t1)


def _check(res, label):
    log(f"[full] {label}: max_err={res['max_err']:.3e} tol={res['tol']} sentinels={res['sentinel_ok']} "
        f"finite={res['finite']} k={np.round(res['k_err'], 4).tolist()} v={np.round(res['v_err'], 4).tolist()}")
    assert res["finite"] and res["sentinel_ok"] and res["max_err"] <= res["tol"], label


@pytest.mark.timeout(300)
def test_fill_llama8b_shaped_full():
    cfg = synth.C2
    sample = _boundary_sample(0, cfg.fill_t1, cfg.fill_chunk, 21)
    _check(run_fill_case(FillCase(cfg, 0, cfg.fill_t1, maps="law", sample=sample, gen_device="cuda")),
           "d4096 x16 layers T16384")


@pytest.mark.timeout(300)
def test_fill_27b_shaped_exact_prefix_and_tail():
    cfg = synth.C3
    sample = _boundary_sample(cfg.fill_t0, cfg.fill_t1, cfg.fill_chunk, 22)
    _check(run_fill_case(FillCase(cfg, cfg.fill_t0, cfg.fill_t1, sample=sample, gen_device="cuda",
                                  max_tokens=cfg.prompt_tokens)), "d5120 x48 layers [2048,28672)")


@pytest.mark.timeout(300)
def test_fill_long_context_paged_chunks():
    cfg = synth.C5
    sample = _boundary_sample(0, cfg.fill_t1, cfg.fill_chunk, 23)
    _check(run_fill_case(FillCase(cfg, 0, cfg.fill_t1, chunk=cfg.fill_chunk, sample=sample, gen_device="cuda",
                                  max_tokens=cfg.prompt_tokens)), "d4096 x16 layers paged T131072")


def _fit_full(cfg, lambdas, n_cols_per_layer=3, seed=0):
    import linear_kv_cache_amd as rf
    from linear_kv_cache_amd.runner import GramState, device_bytes
    dev = "cuda"
    L, d = cfg.n_targets, cfg.d
    rng = np.random.default_rng(seed)
    cols = [np.sort(rng.choice(d, n_cols_per_layer, replace=False)) for _ in range(L)]
    st = GramState(d, L, cfg.torch_dtype, dev)
    Xh, Yh = [], [[] for _ in range(L)]
    n_chunks = cfg.calib_rows // cfg.calib_chunk
    for c in range(n_chunks):
        Xc = synth.hidden_states(cfg, cfg.calib_chunk, "calib", chunk=c, device=dev)
        Ys = [synth.late_layer_inputs(cfg, Xc, l, chunk=c) for l in cfg.filled_layers]
        st.accumulate(Xc, Ys)
        Xh.append(Xc.cpu())
        for l in range(L):
            Yh[l].append(Ys[l][:, torch.as_tensor(cols[l], device=dev)].cpu())
        del Ys
    torch.cuda.synchronize()
    log(f"[full-fit] accumulated {n_chunks} chunks; copying the state")
    S_xx, S_yx = f64(st.S_xx()), st.S_yx()
    s_x, s_y, n = f64(st.s_x()), f64(st.s_y()), int(st.n().item())
    X = torch.cat(Xh).float().numpy().astype(np.float64)
    Ysel = [torch.cat(y).float().numpy().astype(np.float64) for y in Yh]
    assert n == X.shape[0]
    # sampled Gram entries against exact fp64 sums
    ii = rng.integers(0, d, 64)
    jj = rng.integers(0, d, 64)
    lo, hi = np.minimum(ii, jj), np.maximum(ii, jj)
    ref_xx = np.einsum("ri,ri->i", X[:, lo], X[:, hi])
    scale_xx = np.max(np.abs(np.einsum("ri,ri->i", X[:, :64], X[:, :64])))
    e_xx = np.max(np.abs(S_xx[lo, hi] - ref_xx)) / scale_xx
    e_sx = np.max(np.abs(s_x - X.sum(0))) / np.max(np.abs(X.sum(0)))
    e_yx, e_sy = 0.0, 0.0
    for l in range(L):
        g = f64(S_yx[l][torch.as_tensor(cols[l], device=dev)])   # [n_cols, d]
        ref = Ysel[l].T @ X
        e_yx = max(e_yx, np.max(np.abs(g - ref)) / np.max(np.abs(ref)))
        e_sy = max(e_sy, np.max(np.abs(s_y[l][cols[l]] - Ysel[l].sum(0))) / np.max(np.abs(Ysel[l].sum(0))))
    log(f"[full-fit] {cfg.name} gram: e_xx={e_xx:.2e} e_yx={e_yx:.2e} e_sx={e_sx:.2e} e_sy={e_sy:.2e}")
    assert e_xx <= 1e-5 and e_yx <= 1e-5 and e_sx <= 1e-12 and e_sy <= 1e-12
    # oracle: the exact one-pass sums of the data (the full Gram once, the sampled target
    # columns of every layer), then the oracle's solve from those sums for every lambda
    # (column j of W depends only on column j of Y)
    sums = oracle.gram_sums(X, Ysel)
    ws = device_bytes(rf.rf_solve_workspace_bytes(st.desc, L), dev)
    for lam in lambdas:
        W, _, b, info = st.solve(lam, rf.RF_LAMBDA_ABSOLUTE, list(range(L)), want_bf16=False, ws=ws)
        torch.cuda.synchronize()
        assert int(info.item()) == 0
        refs = oracle.fit_from_sums(*sums, lam)
        errs, berrs = [], []
        for l, (Wref, bref) in enumerate(refs):
            Wg = f64(W[l][torch.as_tensor(cols[l], device=dev)]).T   # [d, n_cols]
            errs.append(np.max(np.abs(Wg - Wref)) / np.max(np.abs(Wref)))
            berrs.append(np.max(np.abs(f64(b[l])[cols[l]] - bref)) / max(np.max(np.abs(bref)), 1e-30))
        log(f"[full-fit] {cfg.name} lambda={lam}: W_err max={max(errs):.2e} b_err max={max(berrs):.2e}")
        assert max(errs) <= W_TOL and max(berrs) <= W_TOL


@pytest.mark.timeout(600)
def test_fit_llama8b_shaped_full():
    _fit_full(synth.C2, synth.C2.lambdas)


@pytest.mark.timeout(900)
def test_fit_heavy_three_lambdas_full():
    _fit_full(synth.C4, synth.C4.lambdas)
