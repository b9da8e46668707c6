"""End to end: the solve's packed bf16 maps and bias feed the fill directly (the benchmark's
pipeline), against the oracle's fit followed by the oracle's fill of the same prompt."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_cases import KV_TOL_BF16, FitCase, f64, log, run_fit_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_fit_then_fill_with_the_solve_s_packed_maps():
    import linear_kv_cache_amd as rf
    from linear_kv_cache_amd.runner import Filler, alloc_cache, gather_rows, pack_weights
    cfg = synth.scaled(synth.C2, name="pipeline-d512", d=512, n_layers=6, split=3, n_kv_heads=2, head_dim=128)
    case = FitCase(cfg, 4000, [2500, 1500], 1e-1)
    res = run_fit_case(case)
    assert res["info"] == 0
    nt = len(res["Ys"])
    layers = [cfg.split + l for l in range(nt)]
    kv = [synth.kv_weights(cfg, l, device="cuda") for l in layers]
    fw = rf.FillWeights(cfg.d, cfg.n_kv_heads, cfg.head_dim, cfg.rms_eps, torch.bfloat16,
                        [res["Wlp"][i] for i in range(nt)], [res["b"][i] for i in range(nt)],
                        [g for (_, _, g) in kv], [pack_weights(k, cfg.head_dim) for (k, _, _) in kv],
                        [pack_weights(v, cfg.head_dim) for (_, v, _) in kv])
    T, pos0 = 600, 11
    X = synth.hidden_states(cfg, T, "prompt", device="cuda")
    cache = alloc_cache(nt, cfg.n_kv_heads, cfg.head_dim, T, torch.bfloat16, "cuda")
    Filler(fw, cfg.rope_base, pos0 + T, T, "cuda").fill(X, 0, T, pos0, cache)
    torch.cuda.synchronize()

    Xc, Xp = f64(res["X"]), f64(X)
    errs = []
    for i, l in enumerate(layers):
        W_ref, b_ref = oracle.fit(Xc, f64(res["Ys"][i]), case.lam, case.mode)
        Wk, Wv, g = kv[i]
        K_ref, V_ref = oracle.fill_layer(Xp, W_ref, b_ref, f64(g), f64(Wk).T, f64(Wv).T,
                                         pos0 + np.arange(T, dtype=np.float64), cfg.n_kv_heads, cfg.head_dim,
                                         cfg.rms_eps, cfg.rope_base)
        K = f64(gather_rows(cache, cache.k[i], 0, T))
        V = f64(gather_rows(cache, cache.v[i], 0, T))
        ke = float(np.max(np.abs(K - K_ref)) / np.sqrt(np.mean(K_ref ** 2)))
        ve = float(np.max(np.abs(V - V_ref)) / np.sqrt(np.mean(V_ref ** 2)))
        log(f"[pipeline] layer {l}: k_err={ke:.3e} v_err={ve:.3e} (tol {KV_TOL_BF16})")
        errs += [ke, ve]
    assert max(errs) <= KV_TOL_BF16
