"""The solve's routes on the GPU: one call for a batch of ridge strengths, the split-bf16 and
fp64 products with the device-side choice between them, and the fp64 stationarity residual.

The ill-conditioned calibration set has the shape the KV-Lingo page reports for trained
caches (appendix B.2, Table 3: low effective rank, strongly anisotropic): a rank-64 mixture
with small isotropic noise and near-duplicate channel pairs, where the equilibrated inverse
carries entries near 80 and the split product alone misses the 1e-3 bar."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_cases import W_TOL, f64, log

pytestmark = pytest.mark.gpu

ILL = synth.scaled(synth.C2, name="lowrank-dups-d512", d=512, n_layers=4, split=2, n_kv_heads=2, head_dim=128)
WELL = synth.scaled(synth.C2, name="gaussian-d512", d=512, n_layers=4, split=2, n_kv_heads=2, head_dim=128)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _state(cfg, X, Ys, chunks):
    from linear_kv_cache_amd.runner import GramState
    st = GramState(cfg.d, len(Ys), cfg.torch_dtype, "cuda")
    Xd, Yd = X.cuda(), [Y.cuda() for Y in Ys]
    r0 = 0
    for c in chunks:
        st.accumulate(Xd[r0:r0 + c], [Y[r0:r0 + c] for Y in Yd])
        r0 += c
    assert r0 == X.shape[0]
    return st


def _sums(st):
    """The state's sums, upcast, with S_xx mirrored from its upper triangle."""
    S = f64(st.S_xx())
    S = np.triu(S) + np.triu(S, 1).T
    return S, f64(st.S_yx()), f64(st.s_x()), f64(st.s_y()), int(st.n().item())


def _errs(W, b, X, Ys, lams):
    ew = np.zeros((len(lams), len(Ys)))
    eb = np.zeros_like(ew)
    for z, lam in enumerate(lams):
        for l, Y in enumerate(Ys):
            W_ref, b_ref = oracle.fit(f64(X), f64(Y), lam)
            ew[z, l] = np.max(np.abs(f64(W[z, l]).T - W_ref)) / np.max(np.abs(W_ref))
            eb[z, l] = np.max(np.abs(f64(b[z, l]) - b_ref)) / max(np.max(np.abs(b_ref)), 1e-30)
    return ew, eb


def test_ill_conditioned_fit_takes_the_fp64_product():
    import linear_kv_cache_amd as rf
    from linear_kv_cache_amd.runner import pack_weights
    X = synth.low_rank_states(ILL, 8192, "calib")
    Ys = [synth.late_layer_inputs(ILL, X, l) for l in ILL.filled_layers[:2]]
    st = _state(ILL, X, Ys, [4096, 4096])
    lams = [1e-3, 1e-1]
    S_xx, S_yx, s_x, s_y, n = _sums(st)
    out = {}
    for name, product in (("auto", rf.RF_PRODUCT_AUTO), ("split", rf.RF_PRODUCT_SPLIT_BF16),
                          ("f64", rf.RF_PRODUCT_F64)):
        W, Wlp, b, info, cond, resid = st.solve_many(lams, 0, [0, 1], product=product, want_resid=True)
        torch.cuda.synchronize()
        assert info.cpu().tolist() == [0, 0]
        ew, eb = _errs(W, b, X, Ys, lams)
        res = f64(resid)
        # the device residual is the oracle's residual of the same maps on the same sums
        for z, lam in enumerate(lams):
            for l in range(2):
                ref = oracle.stationarity_residual_from_sums(S_xx, S_yx[l].T, s_x, s_y[l], n, f64(W[z, l]).T, lam)
                assert abs(res[z, l] - ref) <= 1e-9 + 1e-6 * ref, (name, z, l, res[z, l], ref)
        log(f"[solve] lowrank-dups {name}: cond={f64(cond).round(1).tolist()} W_err={ew.max():.2e} "
            f"b_err={eb.max():.2e} resid={res.max():.2e}")
        out[name] = (W, Wlp, b, f64(cond), ew, eb, res)
    W, Wlp, b, cond, ew, eb, res = out["auto"]
    assert (cond > rf.RF_SPLIT_COND_MAX).all()            # the indicator sees the collinearity
    assert ew.max() <= W_TOL and eb.max() <= W_TOL          # and the fp64 product meets the bar
    assert res.max() <= 1e-6                                # the fp32 rounding of W, no more
    # AUTO wrote exactly what the fp64 route writes, and its bf16 maps are the fp32 maps packed
    assert torch.equal(W, out["f64"][0]) and torch.equal(b, out["f64"][2])
    for z in range(2):
        for l in range(2):
            assert torch.equal(Wlp[z, l].view(torch.int16), pack_weights(W[z, l]).view(torch.int16))
    # the split product alone leaves a residual far above the fp64 one on this data
    assert out["split"][6].min() > 1e2 * res.max()


def test_well_conditioned_fit_keeps_the_split_product():
    import linear_kv_cache_amd as rf
    X = synth.hidden_states(WELL, 6000, "calib")
    Ys = [synth.late_layer_inputs(WELL, X, l) for l in WELL.filled_layers[:2]]
    st = _state(WELL, X, Ys, [2500, 3500])
    lams = [1e-3, 0.1, 10.0]
    W, Wlp, b, info, cond, resid = st.solve_many(lams, 0, [0, 1], want_resid=True)
    Ws, Wlps, bs, _, conds, _ = st.solve_many(lams, 0, [0, 1], product=rf.RF_PRODUCT_SPLIT_BF16)
    W64, _, b64, _, _, resid64 = st.solve_many(lams, 0, [0, 1], product=rf.RF_PRODUCT_F64, want_resid=True)
    torch.cuda.synchronize()
    assert info.cpu().tolist() == [0, 0, 0]
    assert (f64(cond) <= rf.RF_SPLIT_COND_MAX).all()
    # AUTO took the split route: bit for bit the split-only call
    assert torch.equal(W, Ws) and torch.equal(Wlp.view(torch.int16), Wlps.view(torch.int16)) and torch.equal(b, bs)
    ew, eb = _errs(W, b, X, Ys, lams)
    ew64, eb64 = _errs(W64, b64, X, Ys, lams)
    log(f"[solve] gaussian cond={f64(cond).round(3).tolist()} split W_err={ew.max():.2e} resid={f64(resid).max():.2e}; "
        f"fp64 W_err={ew64.max():.2e} resid={f64(resid64).max():.2e}")
    assert ew.max() <= W_TOL and eb.max() <= W_TOL and ew64.max() <= W_TOL and eb64.max() <= W_TOL
    assert f64(resid64).max() <= 1e-6 and f64(resid).max() <= 1e-3


def test_lambda_batch_matches_single_calls_and_isolates_a_failed_pivot():
    # a batch of ridge strengths in one call: each lambda's maps agree with a call of its own
    # (the batch shares the equilibration of its first lambda, so agreement is to rounding),
    # and a lambda whose system is singular reports its own pivot without touching the others
    X = synth.hidden_states(WELL, 5000, "calib")
    X[:, 77] = 0                                         # a dead channel: singular at lambda 0
    Ys = [synth.late_layer_inputs(WELL, X, l) for l in WELL.filled_layers[:2]]
    st = _state(WELL, X, Ys, [5000])
    lams = [0.0, 0.05, 3.0]
    W, _, b, info, _, _ = st.solve_many(lams, 0, [0, 1], want_bf16=False)
    torch.cuda.synchronize()
    got = info.cpu().tolist()
    ref_pivot = None
    try:
        oracle.fit(f64(X), f64(Ys[0]), 0.0)
    except oracle.NotSPD as e:
        ref_pivot = e.pivot
    log(f"[solve] batch info={got} oracle pivot at lambda 0: {ref_pivot}")
    assert got[0] == ref_pivot and got[1:] == [0, 0]
    for z in (1, 2):
        W1, _, b1, info1 = st.solve(lams[z], 0, [0, 1], want_bf16=False)
        torch.cuda.synchronize()
        assert int(info1.item()) == 0
        assert float((W[z] - W1).abs().max() / W1.abs().max()) <= 1e-4
        ew, eb = _errs(W[z:z + 1], b[z:z + 1], X, Ys, [lams[z]])
        assert ew.max() <= W_TOL and eb.max() <= W_TOL
