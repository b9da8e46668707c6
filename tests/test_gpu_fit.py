"""GPU parity of rf_gram_accumulate and rf_solve against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_cases import W_TOL, FitCase, f64, fit_errors, log, run_fit_case

pytestmark = pytest.mark.gpu

SMALL_BF16 = synth.scaled(synth.C2, name="fit-bf16-d512", d=512, n_layers=6, split=3)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _gram_errors(res):
    X, Ys, st = res["X"], res["Ys"], res["state"]
    S_xx, S_xy, s_x, s_y, n = oracle.gram_sums(f64(X), [f64(Y) for Y in Ys])
    up = np.triu(np.ones_like(S_xx, dtype=bool))
    g_xx = f64(st.S_xx())
    e_xx = float(np.max(np.abs(g_xx[up] - S_xx[up])) / np.max(np.abs(S_xx)))
    g_yx = f64(st.S_yx())
    e_yx = max(float(np.max(np.abs(g_yx[l] - S_xy[l].T)) / np.max(np.abs(S_xy[l]))) for l in range(len(Ys)))
    e_sx = float(np.max(np.abs(f64(st.s_x()) - s_x)) / np.max(np.abs(s_x)))
    e_sy = max(float(np.max(np.abs(f64(st.s_y())[l] - s_y[l])) / np.max(np.abs(s_y[l]))) for l in range(len(Ys)))
    return dict(n=int(st.n().item()), n_ref=n, e_xx=e_xx, e_yx=e_yx, e_sx=e_sx, e_sy=e_sy)


def test_fit_tiny_fp32_one_chunk_and_ragged_chunks():
    for chunks in ([4096], [1000, 3000, 96]):
        case = FitCase(synth.C1, 4096, chunks, 1e-2)
        res = run_fit_case(case)
        g = _gram_errors(res)
        ew, eb = fit_errors(res, case)
        log(f"[fit] C1 chunks={chunks} gram={g} W_err={np.max(ew):.3e} b_err={np.max(eb):.3e} info={res['info']}")
        assert res["info"] == 0
        assert g["n"] == g["n_ref"] == 4096
        assert max(g["e_xx"], g["e_yx"]) <= 1e-5 and max(g["e_sx"], g["e_sy"]) <= 1e-12
        assert max(ew) <= W_TOL and max(eb) <= W_TOL


def test_fit_bf16_ragged_rows_and_relative_lambda():
    case = FitCase(SMALL_BF16, 5000, [1024, 1024, 1024, 1024, 904], 1e-1)
    res = run_fit_case(case)
    g = _gram_errors(res)
    ew, eb = fit_errors(res, case)
    log(f"[fit] bf16 d512 gram={g} W_err={np.max(ew):.3e} b_err={np.max(eb):.3e}")
    assert res["info"] == 0 and g["n"] == 5000
    assert max(g["e_xx"], g["e_yx"]) <= 1e-5 and max(g["e_sx"], g["e_sy"]) <= 1e-12
    assert max(ew) <= W_TOL and max(eb) <= W_TOL
    case_r = FitCase(SMALL_BF16, 5000, [5000], 1e-3, mode="rel_mean_diag")
    res_r = run_fit_case(case_r)
    ew, eb = fit_errors(res_r, case_r)
    log(f"[fit] bf16 d512 relative lambda W_err={np.max(ew):.3e} b_err={np.max(eb):.3e}")
    assert res_r["info"] == 0 and max(ew) <= W_TOL and max(eb) <= W_TOL


def test_fit_bf16_widths_not_a_power_of_two_blocks():
    # d / 64 = 12 and 20 diagonal blocks: the triangular inverse joins units of unequal size
    # and carries unpaired ones between levels
    for d in (768, 1280):
        cfg = synth.scaled(synth.C2, name=f"fit-bf16-d{d}", d=d, n_layers=4, split=2)
        case = FitCase(cfg, 3000, [2000, 1000], 1e-1)
        res = run_fit_case(case)
        ew, eb = fit_errors(res, case)
        log(f"[fit] bf16 d{d} W_err={np.max(ew):.3e} b_err={np.max(eb):.3e}")
        assert res["info"] == 0
        assert max(ew) <= W_TOL and max(eb) <= W_TOL


def test_gram_strided_rows_and_no_targets():
    """X as a column slice of a wider buffer (ldx = d + 256), the Y_l as views into one
    layer-major buffer (ldy = L d), a ragged 700-row chunk; and a state with no targets."""
    from linear_kv_cache_amd.runner import GramState
    cfg = SMALL_BF16
    d, L, rows = cfg.d, 3, 700
    X = synth.hidden_states(cfg, rows, "calib", device="cuda")
    Ys = [synth.late_layer_inputs(cfg, X, cfg.split + l) for l in range(L)]
    wide = torch.zeros(rows, d + 256, dtype=X.dtype, device="cuda")
    wide[:, 128:128 + d] = X
    Xv = wide[:, 128:128 + d]
    Yall = torch.cat(Ys, dim=1).contiguous()
    Yv = [Yall[:, l * d:(l + 1) * d] for l in range(L)]
    assert Xv.stride(0) == d + 256 and Yv[0].stride(0) == L * d
    st = GramState(d, L, cfg.torch_dtype, "cuda")
    st.accumulate(Xv, Yv)
    st0 = GramState(d, 0, cfg.torch_dtype, "cuda")
    st0.accumulate(Xv, [])
    torch.cuda.synchronize()
    res = _gram_errors(dict(X=X, Ys=Ys, state=st))
    log(f"[fit] strided rows gram={res}")
    assert res["n"] == rows and max(res["e_xx"], res["e_yx"]) <= 1e-5 and max(res["e_sx"], res["e_sy"]) <= 1e-12
    assert torch.equal(st0.S_xx(), st.S_xx()) and torch.equal(st0.s_x(), st.s_x()) and int(st0.n().item()) == rows


def test_gram_pieces_for_32_bit_offsets():
    """A row stride of 2^20 elements caps one launch at 896 rows (the products address X with
    32-bit byte offsets), so a 2000-row chunk runs as pieces of 896, 896 and 208 rows.  The state
    equals three calls of those sizes on a contiguous copy bit for bit, and the oracle's sums
    within the usual bounds."""
    from linear_kv_cache_amd.runner import GramState
    cfg = SMALL_BF16
    d, L, rows, ld = cfg.d, 2, 2000, 1 << 20
    X = synth.hidden_states(cfg, rows, "calib", device="cuda")
    Ys = [synth.late_layer_inputs(cfg, X, cfg.split + l) for l in range(L)]
    wide = torch.zeros(rows, ld, dtype=X.dtype, device="cuda")   # 4 GiB
    wide[:, ld - d:] = X
    Xv = wide[:, ld - d:]
    assert Xv.stride(0) == ld
    st = GramState(d, L, cfg.torch_dtype, "cuda")
    st.accumulate(Xv, Ys)
    ref = GramState(d, L, cfg.torch_dtype, "cuda")
    for r0, r1 in ((0, 896), (896, 1792), (1792, rows)):
        ref.accumulate(X[r0:r1], [Y[r0:r1] for Y in Ys])
    torch.cuda.synchronize()
    del wide, Xv
    res = _gram_errors(dict(X=X, Ys=Ys, state=st))
    log(f"[fit] 2^20 row stride, pieces: gram={res}")
    assert torch.equal(st.buf, ref.buf)
    assert res["n"] == rows and max(res["e_xx"], res["e_yx"]) <= 1e-5 and max(res["e_sx"], res["e_sy"]) <= 1e-12


def test_fit_not_spd_reports_pivot():
    case = FitCase(synth.C1, 1024, [1024], 0.0, zero_column=77, n_targets=1)
    res = run_fit_case(case)
    with pytest.raises(oracle.NotSPD) as e:
        oracle.fit(f64(res["X"]), f64(res["Ys"][0]), 0.0)
    log(f"[fit] not SPD: gpu info={res['info']} oracle pivot={e.value.pivot}")
    assert res["info"] == e.value.pivot == 78


def test_solve_with_no_targets_reports_the_pivot_only():
    # n_sel = 0: the factorisation runs (its info is the only output) and no map is written
    from linear_kv_cache_amd.runner import GramState
    cfg = synth.C1
    X = synth.hidden_states(cfg, 1024, "calib", device="cuda")
    Ys = [synth.late_layer_inputs(cfg, X, cfg.split)]
    st = GramState(cfg.d, 1, cfg.torch_dtype, "cuda")
    st.accumulate(X, Ys)
    X0 = X.clone()
    X0[:, 77] = 0
    st0 = GramState(cfg.d, 1, cfg.torch_dtype, "cuda")
    st0.accumulate(X0, Ys)
    infos = []
    for state, lam in ((st, 0.0), (st0, 0.0), (st0, 1e-2)):
        W, Wlp, b, info = state.solve(lam, 0, [])
        torch.cuda.synchronize()
        assert W.numel() == 0 and Wlp.numel() == 0 and b.numel() == 0
        infos.append(int(info.item()))
    log(f"[fit] no targets: infos={infos}")
    assert infos == [0, 78, 0]


def test_gram_deterministic_and_resumable():
    import linear_kv_cache_amd as rf
    from linear_kv_cache_amd.runner import GramState
    cfg = SMALL_BF16
    X = synth.hidden_states(cfg, 3000, "calib", device="cuda")
    Ys = [synth.late_layer_inputs(cfg, X, cfg.split + l) for l in range(2)]
    a = GramState(cfg.d, 2, cfg.torch_dtype, "cuda")
    b = GramState(cfg.d, 2, cfg.torch_dtype, "cuda")
    for st in (a, b):
        st.accumulate(X[:1200], [Y[:1200] for Y in Ys])
        st.accumulate(X[1200:], [Y[1200:] for Y in Ys])
    # checkpoint after the first chunk, restore into a fresh state, continue
    c = GramState(cfg.d, 2, cfg.torch_dtype, "cuda")
    c.accumulate(X[:1200], [Y[:1200] for Y in Ys])
    host = c.buf.cpu()
    d = GramState(cfg.d, 2, cfg.torch_dtype, "cuda")
    d.buf.copy_(host.to("cuda"))
    d.accumulate(X[1200:], [Y[1200:] for Y in Ys])
    torch.cuda.synchronize()
    assert torch.equal(a.buf, b.buf)
    assert torch.equal(a.buf, d.buf)


def test_gram_ragged_chunks_and_row_tails():
    """Chunks of 37, 64, 129 and 1000 rows: the products take 64-row k-steps in pairs, so
    every chunk ends in rows that must read as zero; the sums match the oracle over all rows."""
    from linear_kv_cache_amd.runner import GramState
    cfg = SMALL_BF16
    chunks = [37, 64, 129, 1000]
    X = synth.hidden_states(cfg, sum(chunks), "calib", device="cuda")
    Ys = [synth.late_layer_inputs(cfg, X, cfg.split + l) for l in range(2)]
    st = GramState(cfg.d, 2, cfg.torch_dtype, "cuda")
    r0 = 0
    for c in chunks:
        st.accumulate(X[r0:r0 + c], [Y[r0:r0 + c] for Y in Ys])
        r0 += c
    torch.cuda.synchronize()
    res = _gram_errors(dict(X=X, Ys=Ys, state=st))
    log(f"[fit] ragged chunks {chunks} gram={res}")
    assert res["n"] == res["n_ref"] == sum(chunks)
    assert max(res["e_xx"], res["e_yx"]) <= 1e-5 and max(res["e_sx"], res["e_sy"]) <= 1e-12


def _rect_data(d, m, n_targets, rows, dtype, seed):
    # X ~ N(0, 1) rows; Y_l = X A_l + 0.1 E with a planted A_l ~ N(0, 1/d) of shape [d, m]
    g = synth.generator(seed, "rect")
    X = torch.randn(rows, d, generator=g)
    Ys = [(X @ (torch.randn(d, m, generator=g) / d ** 0.5) + 0.1 * torch.randn(rows, m, generator=g)).to(dtype)
          for _ in range(n_targets)]
    return X.to(dtype), Ys


def test_fit_rectangular_maps():
    # maps with more outputs than inputs (fp32, d = 256 -> m = 512) and fewer (bf16, d = 512 ->
    # m = 256), ragged chunks; Gram sums, W and b against the oracle
    from linear_kv_cache_amd.runner import GramState
    for d, m, nt, dtype, chunks, lam, seed in [(256, 512, 2, torch.float32, [1500, 2596], 1e-2, 11),
                                               (512, 256, 3, torch.bfloat16, [1024, 3000, 77], 1e-1, 12)]:
        X, Ys = _rect_data(d, m, nt, sum(chunks), dtype, seed)
        st = GramState(d, nt, dtype, "cuda", d_out=m)
        Xd, Yd = X.cuda(), [Y.cuda() for Y in Ys]
        r0 = 0
        for c in chunks:
            st.accumulate(Xd[r0:r0 + c], [Y[r0:r0 + c] for Y in Yd])
            r0 += c
        W, Wlp, b, info = st.solve(lam, 0, list(range(nt)))
        torch.cuda.synchronize()
        assert int(info.item()) == 0
        S_xx, S_xy, s_x, s_y, n = oracle.gram_sums(f64(X), [f64(Y) for Y in Ys])
        g_yx = f64(st.S_yx())
        e_yx = max(float(np.max(np.abs(g_yx[l] - S_xy[l].T)) / np.max(np.abs(S_xy[l]))) for l in range(nt))
        e_sy = max(float(np.max(np.abs(f64(st.s_y())[l] - s_y[l])) / np.max(np.abs(s_y[l]))) for l in range(nt))
        ew, eb = [], []
        for l in range(nt):
            W_ref, b_ref = oracle.fit(f64(X), f64(Ys[l]), lam)
            ew.append(float(np.max(np.abs(f64(W[l]).T - W_ref)) / np.max(np.abs(W_ref))))
            eb.append(float(np.max(np.abs(f64(b[l]) - b_ref)) / np.max(np.abs(b_ref))))
        log(f"[fit] rectangular d={d} m={m} {dtype}: e_yx={e_yx:.2e} e_sy={e_sy:.2e} W_err={max(ew):.3e} "
            f"b_err={max(eb):.3e}")
        assert int(st.n().item()) == sum(chunks)
        assert e_yx <= 1e-5 and e_sy <= 1e-12
        assert max(ew) <= W_TOL and max(eb) <= W_TOL
        if dtype == torch.bfloat16:
            # the packed bf16 output is the fp32 map rounded, in the packed layout
            from linear_kv_cache_amd.runner import pack_weights
            for l in range(nt):
                assert torch.equal(Wlp[l].view(torch.int16), pack_weights(W[l].to(torch.bfloat16)).view(torch.int16))


R2_TOL = 1e-4   # absolute, on R^2 in [0, 1]: fp32 sums and maps against fp64 on the data


def test_fit_r2_read_off_the_state():
    # targets explained to different degrees (noise 0.3, 1 and 3 times the signal scale), bf16
    # rectangular and fp32 square; absolute and relative lambda; R^2 against the oracle's
    # definition on the data, and the column sums of squares against fp64 sums
    from linear_kv_cache_amd.runner import GramState
    for d, m, dtype, rows, chunks in [(512, 256, torch.bfloat16, 3000, [1000, 2000]),
                                      (256, 256, torch.float32, 2048, [2048])]:
        g = synth.generator(21, "r2", d, m)
        X = torch.randn(rows, d, generator=g) * (1 + torch.rand(d, generator=g))
        Ys = [X @ (torch.randn(d, m, generator=g) / d ** 0.5) + s * torch.randn(rows, m, generator=g)
              for s in (0.3, 1.0, 3.0)]
        X = X.to(dtype)
        Ys = [Y.to(dtype) for Y in Ys]
        st = GramState(d, 3, dtype, "cuda", d_out=m)
        r0 = 0
        for c in chunks:
            st.accumulate(X[r0:r0 + c].cuda(), [Y[r0:r0 + c].cuda() for Y in Ys])
            r0 += c
        syy = f64(st.s_yy())
        for l, Y in enumerate(Ys):
            ref = np.sum(f64(Y) ** 2, axis=0)
            assert float(np.max(np.abs(syy[l] - ref) / ref)) <= 1e-12
        for lam, mode, mname in [(0.1, 0, "absolute"), (1e-2, 1, "rel_mean_diag")]:
            W, _, _, info = st.solve(lam, mode, [0, 1, 2], want_bf16=False)
            r2 = f64(st.r2(lam, mode, [0, 1, 2], W))
            torch.cuda.synchronize()
            ref = [oracle.fit_r2(f64(X), f64(Y), lam, mname) for Y in Ys]
            log(f"[fit] R^2 d={d} m={m} {dtype} {mname}: gpu={np.round(r2, 6)} oracle={np.round(ref, 6)}")
            assert int(info.item()) == 0
            assert float(np.max(np.abs(r2 - np.array(ref)))) <= R2_TOL
            assert ref[0] > ref[1] > ref[2]


def test_gram_select_equals_a_pass_over_the_selected_columns():
    # the sub-state of blocks [1, 3] of a 4-block X equals the state one pass over those columns
    # alone leaves (the same tile products over the same rows: bit for bit)
    from linear_kv_cache_amd.runner import GramState
    import linear_kv_cache_amd as rf
    g = synth.generator(51, "select")
    n, bw = 2000, 256
    X = torch.randn(n, 4 * bw, generator=g).to(torch.bfloat16).cuda()
    Ys = [torch.randn(n, 512, generator=g).to(torch.bfloat16).cuda() for _ in range(2)]
    full = GramState(4 * bw, 2, torch.bfloat16, "cuda", d_out=512)
    full.accumulate(X, Ys)
    sub = GramState(2 * bw, 2, torch.bfloat16, "cuda", d_out=512)
    rf.rf_gram_select(full.desc, full.buf, bw, [1, 3], sub.desc, sub.buf)
    direct = GramState(2 * bw, 2, torch.bfloat16, "cuda", d_out=512)
    Xs = torch.cat([X[:, bw:2 * bw], X[:, 3 * bw:]], dim=1).contiguous()
    direct.accumulate(Xs, Ys)
    torch.cuda.synchronize()
    up = torch.triu(torch.ones(2 * bw, 2 * bw, dtype=torch.bool)).cuda()
    assert int(sub.n().item()) == int(direct.n().item()) == n
    assert torch.equal(sub.S_xx()[up], direct.S_xx()[up])
    assert torch.equal(sub.S_yx(), direct.S_yx())
    assert torch.equal(sub.s_x(), direct.s_x()) and torch.equal(sub.s_y(), direct.s_y())
    assert torch.equal(sub.s_yy(), direct.s_yy())


def test_fit_pinv_route_regular_and_rank_deficient():
    # the eigendecomposition route: with lambda = 0 on rank-deficient rows (duplicated and
    # constant columns: rf_solve reports a failed pivot) it gives the minimum-norm
    # least-squares map of the oracle; on a regular system (the exact duplicates alone, at the
    # workloads' lambda = 0.1) it gives rf_solve's map.  The duplicates leave the equilibrated
    # inverse entries ~ n var / lambda, so both routes take the fp64 product there.
    from linear_kv_cache_amd.runner import GramState
    g = synth.generator(61, "pinv")
    n, d = 3000, 256
    base = torch.randn(n, 200, generator=g) * (0.5 + torch.rand(200, generator=g))
    X = torch.cat([base, base[:, :40], torch.full((n, 16), 2.0)], dim=1).to(torch.bfloat16)   # rank 200 of 256
    Xr = torch.cat([base, base[:, :40], torch.randn(n, 16, generator=g)], dim=1).to(torch.bfloat16)   # duplicates only
    Ys = [(base @ (torch.randn(200, d, generator=g) / 15) + 0.1 * torch.randn(n, d, generator=g)).to(torch.bfloat16)
          for _ in range(2)]
    for Xs, lam, label in ((X, 0.0, "rank-deficient, lambda 0"), (Xr, 0.1, "duplicated columns, lambda 0.1")):
        st = GramState(d, 2, torch.bfloat16, "cuda")
        st.accumulate(Xs.cuda(), [Y.cuda() for Y in Ys])
        W, _, b = st.solve_pinv(lam, 0, [0, 1])
        torch.cuda.synchronize()
        ew, eb = [], []
        for l in range(2):
            W_ref, b_ref = oracle.fit_pinv(f64(Xs), f64(Ys[l]), lam)
            ew.append(float(np.max(np.abs(f64(W[l]).T - W_ref)) / np.max(np.abs(W_ref))))
            eb.append(float(np.max(np.abs(f64(b[l]) - b_ref)) / max(np.max(np.abs(b_ref)), 1e-30)))
        log(f"[fit] pseudo-inverse route, {label}: W_err={max(ew):.3e} b_err={max(eb):.3e}")
        assert max(ew) <= W_TOL and max(eb) <= W_TOL
        if lam > 0:
            W2, _, b2, info, cond, _ = st.solve_many([lam], 0, [0, 1], want_bf16=False)
            torch.cuda.synchronize()
            assert int(info.item()) == 0
            log(f"[fit] Cholesky route on the same system: cond={float(cond.item()):.3e}")
            assert float(cond.item()) > 8.0
            assert float((W2[0] - W).abs().max() / W2[0].abs().max()) <= W_TOL
            for l in range(2):
                W_ref, _ = oracle.fit(f64(Xs), f64(Ys[l]), lam)
                assert float(np.max(np.abs(f64(W2[0, l]).T - W_ref)) / np.max(np.abs(W_ref))) <= W_TOL
        else:
            _, _, _, info = st.solve(0.0, 0, [0], want_bf16=False)
            torch.cuda.synchronize()
            assert int(info.item()) > 0          # the Cholesky route cannot factor the singular system
