"""Host-side checks of the C ABI: the library loads, exports every declared symbol, and its
host-only arithmetic and argument validation behave as the header says.  No kernel is
launched here (every call below returns before any enqueue)."""
import ctypes as C
import os
import re

import pytest
import torch

import linear_kv_cache_amd as rf

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "ridgefill.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rf_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 12
    lib = C.CDLL(rf.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(rf.EXPORTED)
    assert rf.rf_version().startswith("ridgefill")


def test_cache_layout_contiguous_and_paged():
    d = rf.cache_desc(8, 128, 1000, rf.RF_LAYOUT_CONTIGUOUS, torch.bfloat16)
    L = rf.rf_cache_layout(d)
    assert L == dict(n_blocks=1000, elem_bytes=2, bytes_per_pool=1000 * 8 * 128 * 2, stride_block=0,
                     stride_head=128, stride_token=1024)
    p = rf.cache_desc(8, 128, 1000, rf.RF_LAYOUT_PAGED, torch.bfloat16, block_size=16)
    L = rf.rf_cache_layout(p)
    assert L["n_blocks"] == 63 and L["stride_block"] == 8 * 16 * 128
    assert L["stride_head"] == 16 * 128 and L["stride_token"] == 128
    assert L["bytes_per_pool"] == 63 * 8 * 16 * 128 * 2
    f = rf.cache_desc(4, 64, 512, rf.RF_LAYOUT_CONTIGUOUS, torch.float32)
    assert rf.rf_cache_layout(f)["elem_bytes"] == 4


def test_cache_layout_rejects_bad_descriptors():
    with pytest.raises(rf.RidgeFillError) as e:
        rf.rf_cache_layout(rf.cache_desc(0, 128, 10, rf.RF_LAYOUT_CONTIGUOUS, torch.bfloat16))
    assert e.value.status == rf.RF_ERR_INVALID_ARG
    with pytest.raises(rf.RidgeFillError):
        rf.rf_cache_layout(rf.cache_desc(8, 128, 10, rf.RF_LAYOUT_PAGED, torch.bfloat16, block_size=0))


def test_gram_state_layout():
    desc = rf.gram_desc(4096, 16, torch.bfloat16)
    L = rf.rf_gram_state_layout(desc)
    assert L["off_n"] == 0 and L["off_S_xx"] == 256
    assert L["off_S_yx"] == 256 + 4096 * 4096 * 4
    assert L["off_s_x"] == L["off_S_yx"] + 16 * 4096 * 4096 * 4
    assert L["off_s_y"] == L["off_s_x"] + 4096 * 8
    assert L["off_s_yy"] == L["off_s_y"] + 16 * 4096 * 8
    assert L["total_bytes"] == L["off_s_yy"] + 16 * 4096 * 8
    assert all(v % 256 == 0 for v in L.values())
    assert rf.rf_gram_state_bytes(desc) == L["total_bytes"]
    assert rf.rf_gram_state_bytes(rf.gram_desc(100, 2, torch.float32)) == 0


def test_gram_state_layout_rectangular_maps():
    # d_out = 1024 outputs per target from d = 2048 inputs (e.g. a translator reading two
    # source layers): S_yx is [n_targets * 1024][2048], s_y [n_targets * 1024]
    desc = rf.gram_desc(2048, 3, torch.bfloat16, d_out=1024)
    L = rf.rf_gram_state_layout(desc)
    assert L["off_S_yx"] == 256 + 2048 * 2048 * 4
    assert L["off_s_x"] == L["off_S_yx"] + 3 * 1024 * 2048 * 4
    assert L["off_s_yy"] == L["off_s_y"] + 3 * 1024 * 8
    assert L["total_bytes"] == L["off_s_yy"] + 3 * 1024 * 8
    assert rf.rf_gram_state_layout(rf.gram_desc(512, 2, torch.float32, d_out=512)) == \
        rf.rf_gram_state_layout(rf.gram_desc(512, 2, torch.float32))
    for d_out, status in ((300, rf.RF_ERR_UNSUPPORTED), (-256, rf.RF_ERR_INVALID_ARG)):
        with pytest.raises(rf.RidgeFillError) as e:
            rf.rf_gram_state_layout(rf.gram_desc(512, 1, torch.float32, d_out=d_out))
        assert e.value.status == status
    assert rf.rf_solve_workspace_bytes(rf.gram_desc(512, 1, torch.float32, d_out=300), 1) == 0
    assert rf.rf_solve_workspace_bytes(rf.gram_desc(512, 2, torch.float32, d_out=1024), 2) > \
        rf.rf_solve_workspace_bytes(rf.gram_desc(512, 2, torch.float32), 2)
    # Y rows shorter than d_out are refused before anything is enqueued
    ys = (C.c_void_p * 1)(256)
    with pytest.raises(rf.RidgeFillError) as e:
        rf._check(rf._lib.rf_gram_accumulate(C.byref(rf.gram_desc(256, 1, torch.float32, d_out=512)), 256, 256, 256,
                                             ys, 256, 4, None))
    assert e.value.status == rf.RF_ERR_INVALID_ARG


def test_gram_validation_before_enqueue():
    with pytest.raises(rf.RidgeFillError) as e:
        rf.rf_gram_init(rf.gram_desc(300, 1, torch.float32), 256, None)
    assert e.value.status == rf.RF_ERR_UNSUPPORTED
    desc = rf.gram_desc(256, 1, torch.float32)
    with pytest.raises(rf.RidgeFillError) as e:
        rf.rf_gram_init(desc, 255, None)  # misaligned state pointer
    assert e.value.status == rf.RF_ERR_INVALID_ARG
    X = torch.empty(4, 256)
    with pytest.raises(rf.RidgeFillError):
        rf.rf_gram_accumulate(desc, 256, X, [], rows=-1)
    with pytest.raises(rf.RidgeFillError) as e:
        rf.rf_gram_accumulate(rf.gram_desc(256, 65, torch.float32), 256, X, [])
    assert e.value.status == rf.RF_ERR_UNSUPPORTED
    rf.rf_gram_accumulate(desc, 256, X, [X], rows=0)  # zero rows: a no-op
    # bf16 rows: pointers and strides are checked before anything is enqueued
    db = rf.gram_desc(256, 1, torch.bfloat16)
    ys = (C.c_void_p * 1)(256)
    for X_ptr, ldx, ldy in ((264, 256, 256), (256, 200, 256), (256, 256, 260), (0, 256, 256)):
        with pytest.raises(rf.RidgeFillError) as e:
            rf._check(rf._lib.rf_gram_accumulate(C.byref(db), 256, X_ptr, ldx, ys, ldy, 4, None))
        assert e.value.status == rf.RF_ERR_INVALID_ARG
    with pytest.raises(rf.RidgeFillError) as e:   # a null Y pointer
        rf._check(rf._lib.rf_gram_accumulate(C.byref(db), 256, 256, 256, (C.c_void_p * 1)(0), 256, 4, None))
    assert e.value.status == rf.RF_ERR_INVALID_ARG


def test_solve_validation_before_enqueue():
    desc = rf.gram_desc(256, 2, torch.float32)
    ws_bytes = rf.rf_solve_workspace_bytes(desc, 2)
    assert ws_bytes > 2 * 256 * 256 * 8
    # each extra lambda of a batch adds its own factor and inverse (2 d^2 fp64) and little else
    assert rf.rf_solve_workspace_bytes(desc, 2, 3) - ws_bytes >= 2 * 2 * 256 * 256 * 8
    assert rf.rf_solve_workspace_bytes(desc, 2, 0) == 0 and rf.rf_solve_workspace_bytes(desc, 2, 9) == 0

    def call(lams, targets, product=0, W=None, resid=None):
        la = (C.c_double * max(1, len(lams)))(*lams)
        rf._check(rf._lib.rf_solve(C.byref(desc), 256, la, len(lams), 0, (C.c_int32 * 1)(*targets), len(targets),
                                   product, W, None, None, 512, None, resid, 256, 16, None))

    for lams, targets, kw, status in [([-1.0], [0], {}, rf.RF_ERR_INVALID_ARG),
                                      ([float("nan")], [0], {}, rf.RF_ERR_INVALID_ARG),
                                      ([0.1, -1.0], [0], {}, rf.RF_ERR_INVALID_ARG),
                                      ([], [0], {}, rf.RF_ERR_INVALID_ARG),
                                      ([0.1] * 9, [0], {}, rf.RF_ERR_INVALID_ARG),
                                      ([0.1], [2], {}, rf.RF_ERR_INVALID_ARG),
                                      ([0.1], [0], dict(product=3), rf.RF_ERR_INVALID_ARG),
                                      ([0.1], [0], dict(resid=1024), rf.RF_ERR_INVALID_ARG),   # residual needs W
                                      ([0.1], [0], {}, rf.RF_ERR_WORKSPACE),
                                      ([1e-3, 0.1, 10.0], [0], dict(W=256, resid=1024), rf.RF_ERR_WORKSPACE)]:
        with pytest.raises(rf.RidgeFillError) as e:
            call(lams, targets, **kw)
        assert e.value.status == status, (lams, targets, kw)


def test_info_status_host():
    assert rf.rf_info_status([0, 0, 0]) == rf.RF_OK
    assert rf.rf_info_status([]) == rf.RF_OK
    assert rf.rf_info_status([0, 78, 0]) == rf.RF_ERR_NOT_SPD
    assert "lambda 1" in rf.rf_last_error() and "78" in rf.rf_last_error()


def _weights(d=256, H=4, dh=64, dtype=torch.float32, n=1, ptr=256):
    return rf.FillWeights(d, H, dh, 1e-6, dtype, [ptr] * n, [ptr] * n, [ptr] * n, [ptr] * n, [ptr] * n)


def _weights_kn(eps, ptr=256):
    w = _weights()
    w.k_norm, w.k_norm_eps = [ptr], eps
    return w


def _weights_q8(ptr=256, dtype=torch.float32):
    w = _weights(dtype=dtype)
    w.map_scale = [ptr]
    return w


def _aligned_bytes(n, a=256):
    buf = torch.empty(n + a, dtype=torch.uint8)
    off = (-buf.data_ptr()) % a
    return buf[off:off + n]


def test_fill_validation_before_enqueue():
    cache = rf.cache_desc(4, 64, 512, rf.RF_LAYOUT_CONTIGUOUS, torch.float32)
    X = torch.empty(512, 256)
    ws = _aligned_bytes(1 << 20)
    rope = torch.empty(512, 64)

    def call(w=None, t0=0, t1=512, pos0=0, cache_=cache, rope_len=512, ws_=ws, n_layers=None, rope_=rope):
        w = w or _weights()
        rf.rf_fill(w, X, t0, t1, pos0, cache_, [256], [256], None, rope_, rope_len, ws_, None, n_layers=n_layers)

    def based(base):
        w = _weights()
        w.rope_base = base
        return w

    need = rf.rf_fill_workspace_bytes(_weights(), 512)
    assert rf.rf_rope_workspace_bytes(64, 512) == 512 * 64 * 4

    cases = [
        (dict(t0=5, t1=4), rf.RF_ERR_INVALID_ARG),
        (dict(w=_weights(d=320)), rf.RF_ERR_UNSUPPORTED),
        (dict(w=_weights(dh=96, H=8)), rf.RF_ERR_UNSUPPORTED),
        (dict(w=_weights(dtype=torch.bfloat16)), rf.RF_ERR_UNSUPPORTED),
        (dict(t1=513), rf.RF_ERR_INVALID_ARG),
        (dict(pos0=1), rf.RF_ERR_INVALID_ARG),  # rope table too short
        (dict(w=_weights_kn(-1.0)), rf.RF_ERR_INVALID_ARG),   # negative key-norm epsilon
        (dict(w=_weights_kn(1e-6, ptr=0)), rf.RF_ERR_INVALID_ARG),   # null key-norm weights
        (dict(ws_=_aligned_bytes(256)), rf.RF_ERR_WORKSPACE),
        (dict(cache_=rf.cache_desc(4, 64, 512, rf.RF_LAYOUT_PAGED, torch.float32)), rf.RF_ERR_INVALID_ARG),
        (dict(w=_weights_q8(ptr=256)), rf.RF_ERR_UNSUPPORTED),    # int8 maps need bf16 weights
        (dict(rope_=None), rf.RF_ERR_INVALID_ARG),                 # no table and no rope_base
        (dict(rope_=None, w=based(float("inf"))), rf.RF_ERR_INVALID_ARG),
        (dict(rope_=None, w=based(1e4), ws_=_aligned_bytes(need)), rf.RF_ERR_WORKSPACE),   # no room for the table
    ]
    for kw, status in cases:
        with pytest.raises(rf.RidgeFillError) as e:
            call(**kw)
        assert e.value.status == status, kw
    call(t0=7, t1=7)          # empty range: nothing to do
    call(n_layers=0)          # no layers: nothing to do
    assert rf.rf_fill_workspace_bytes(_weights(), 512) >= 512 * 256 * 4


def test_rope_table_validation():
    for args in [(0.0, 64, 10), (1e4, 63, 10), (1e4, 64, -1)]:
        with pytest.raises(rf.RidgeFillError):
            rf.rf_rope_table(*args, 256, None)
    rf.rf_rope_table(1e4, 64, 0, 256, None)  # zero positions: nothing to do


def test_pack_weights_validation_before_enqueue():
    bf = torch.bfloat16
    src = torch.zeros(256, 128, dtype=bf)
    dst = torch.zeros(256, 128, dtype=bf)
    cases = [
        (dict(W=src[:100], dst=dst), rf.RF_ERR_UNSUPPORTED),                  # rows % 256
        (dict(W=src[:, :100], dst=dst), rf.RF_ERR_UNSUPPORTED),               # cols % 64
        (dict(W=src, dst=dst, rope_head_dim=32), rf.RF_ERR_UNSUPPORTED),
        (dict(W=torch.zeros(256, 68, dtype=bf)[:, :64], dst=dst), rf.RF_ERR_INVALID_ARG),  # stride % 8
        (dict(W=src, dst=None), rf.RF_ERR_INVALID_ARG),
        (dict(W=src, dst=dst.data_ptr() + 2), rf.RF_ERR_INVALID_ARG),         # misaligned output
    ]
    for kw, status in cases:
        with pytest.raises(rf.RidgeFillError) as e:
            rf.rf_pack_weights(stream=0, **kw)
        assert e.value.status == status, kw
    rf.rf_pack_weights(src[:0], dst, stream=0)   # no rows: nothing to do
    with pytest.raises(rf.RidgeFillError) as e:    # an element type that is neither BF16 nor F32
        rf._check(rf._lib.rf_pack_weights(7, 256, 128, src.data_ptr(), 128, 0, dst.data_ptr(), None))
    assert e.value.status == rf.RF_ERR_UNSUPPORTED


def test_quantize_map_validation_before_enqueue():
    W = torch.zeros(256, 128)
    q = torch.zeros(256 * 128, dtype=torch.int8)
    s = torch.zeros(256)
    cases = [
        (dict(W=W[:100], q=q, scale=s), rf.RF_ERR_UNSUPPORTED),               # rows % 256
        (dict(W=W[:, :100], q=q, scale=s), rf.RF_ERR_UNSUPPORTED),            # cols % 64
        (dict(W=torch.zeros(256, 66)[:, :64], q=q, scale=s), rf.RF_ERR_INVALID_ARG),   # stride % 4
        (dict(W=W, q=None, scale=s), rf.RF_ERR_INVALID_ARG),
        (dict(W=W, q=q.data_ptr() + 8, scale=s), rf.RF_ERR_INVALID_ARG),     # misaligned codes
    ]
    for kw, status in cases:
        with pytest.raises(rf.RidgeFillError) as e:
            rf.rf_quantize_map(stream=0, **kw)
        assert e.value.status == status, kw
    rf.rf_quantize_map(W[:0], q, s, stream=0)   # no rows: nothing to do


def test_relative_depth_sources_matches_the_oracle():
    # host arithmetic, compared exactly with the oracle's nearest-band search
    import oracle
    for n_src in (1, 2, 3, 5, 12, 28, 36, 64):
        for n_tgt in (1, 2, 3, 5, 17, 28, 36, 64):
            for nu in sorted({1, 2, 3, 4, n_src} & set(range(1, n_src + 1))):
                assert rf.rf_relative_depth_sources(n_src, n_tgt, nu) == \
                    oracle.relative_depth_sources(n_src, n_tgt, nu), (n_src, n_tgt, nu)
    for bad in [(4, 4, 5), (4, 0, 1), (4, 4, 0)]:
        with pytest.raises(rf.RidgeFillError) as e:
            rf.rf_relative_depth_sources(*bad)
        assert e.value.status == rf.RF_ERR_INVALID_ARG


def _tweights(d_in=256, H=4, dh=64, dtype=torch.float32, n=1, ptr=256, bias=False):
    b = [ptr] * n if bias else None
    return rf.TranslateWeights(d_in, H, dh, dtype, [ptr] * n, [ptr] * n, b, b)


def test_translate_validation_before_enqueue():
    cache = rf.cache_desc(4, 64, 512, rf.RF_LAYOUT_CONTIGUOUS, torch.float32)
    rope = torch.empty(512, 64)

    def call(w=None, t0=0, t1=512, pos0=0, cache_=cache, rope_len=512, ld=256, src=256, n_layers=None):
        w = w or _tweights()
        rf.rf_translate(w, [src], [src], ld, t0, t1, pos0, cache_, [256], [256], None, rope, rope_len,
                        n_layers=n_layers)

    w_half_bias = _tweights()
    w_half_bias.b_k = [256]
    w_kn_eps = _tweights()
    w_kn_eps.k_norm, w_kn_eps.k_norm_eps = [256], -1.0
    w_kn_null = _tweights()
    w_kn_null.k_norm = [0]
    cases = [
        (dict(t0=5, t1=4), rf.RF_ERR_INVALID_ARG),
        (dict(w=_tweights(d_in=96)), rf.RF_ERR_UNSUPPORTED),                 # F32: d_in % 64
        (dict(w=_tweights(d_in=192, dtype=torch.bfloat16)), rf.RF_ERR_UNSUPPORTED),  # BF16: % 128
        (dict(w=_tweights(dh=96, H=8)), rf.RF_ERR_UNSUPPORTED),
        (dict(w=_tweights(H=2)), rf.RF_ERR_UNSUPPORTED),                     # K width % 256
        (dict(t1=513, rope_len=600), rf.RF_ERR_INVALID_ARG),                 # past max_tokens
        (dict(pos0=1), rf.RF_ERR_INVALID_ARG),                               # rope table too short
        (dict(ld=200), rf.RF_ERR_INVALID_ARG),                               # ld_src < d_in
        (dict(ld=257), rf.RF_ERR_INVALID_ARG),                               # ld_src not 16-byte
        (dict(src=260), rf.RF_ERR_INVALID_ARG),                              # misaligned source
        (dict(src=0), rf.RF_ERR_INVALID_ARG),
        (dict(w=w_half_bias), rf.RF_ERR_INVALID_ARG),                        # only b_k given
        (dict(w=w_kn_eps), rf.RF_ERR_INVALID_ARG),                           # negative key-norm epsilon
        (dict(w=w_kn_null), rf.RF_ERR_INVALID_ARG),                          # null key-norm weights
        (dict(cache_=rf.cache_desc(4, 64, 512, rf.RF_LAYOUT_PAGED, torch.float32)), rf.RF_ERR_INVALID_ARG),
    ]
    for kw, status in cases:
        with pytest.raises(rf.RidgeFillError) as e:
            call(**kw)
        assert e.value.status == status, kw
    call(t0=7, t1=7)          # empty range: nothing to do
    call(n_layers=0)          # no layers: nothing to do


def test_r2_assignment_matches_the_oracle():
    # host ranking, compared exactly with the oracle's (ties and NaN included)
    import numpy as np
    import oracle
    g = np.random.default_rng(0)
    cases = [np.array([[0.1, 0.9, 0.5, 0.9], [0.8, 0.2, 0.8, 0.3], [0.0, 0.0, 0.0, 0.0]]),
             np.array([[np.nan, 0.5, 0.4], [0.3, np.nan, np.nan]]),
             g.random((36, 28)), np.round(g.random((12, 9)), 1)]
    for r2 in cases:
        for nu in range(1, r2.shape[1] + 1):
            assert rf.rf_r2_assignment(r2.tolist(), nu) == oracle.r2_assignment(r2, nu), (r2.shape, nu)
    with pytest.raises(rf.RidgeFillError) as e:
        rf.rf_r2_assignment([[0.5, 0.2]], 3)
    assert e.value.status == rf.RF_ERR_INVALID_ARG


def test_fit_r2_validation_before_enqueue():
    desc = rf.gram_desc(256, 2, torch.float32)
    assert rf.rf_fit_r2_workspace_bytes(desc, 2) >= 2 * (256 // 16) * 2 * 8
    ws = _aligned_bytes(1 << 16)
    r2 = _aligned_bytes(64)
    for lam, targets, status in [(-1.0, [0], rf.RF_ERR_INVALID_ARG), (0.1, [2], rf.RF_ERR_INVALID_ARG),
                                 (0.1, [0] * 65, rf.RF_ERR_UNSUPPORTED)]:
        with pytest.raises(rf.RidgeFillError) as e:
            rf.rf_fit_r2(desc, 256, lam, 0, targets, 256, r2, ws, stream=0)
        assert e.value.status == status, (lam, targets)
    with pytest.raises(rf.RidgeFillError) as e:
        rf.rf_fit_r2(desc, 256, 0.1, 0, [0], 256, r2, _aligned_bytes(128), stream=0)
    assert e.value.status == rf.RF_ERR_WORKSPACE
    rf.rf_fit_r2(desc, 256, 0.1, 0, [], 256, r2, ws, stream=0)   # nothing selected: nothing to do


def test_gram_select_validation_before_enqueue():
    src = rf.gram_desc(1024, 2, torch.bfloat16, d_out=512)
    ok = rf.gram_desc(512, 2, torch.bfloat16, d_out=512)
    cases = [
        (dict(bw=300, blocks=[0]), rf.RF_ERR_UNSUPPORTED),                    # width not a multiple of 256
        (dict(bw=768, blocks=[0]), rf.RF_ERR_UNSUPPORTED),                    # does not divide d
        (dict(bw=256, blocks=[2, 1]), rf.RF_ERR_INVALID_ARG),                 # not ascending
        (dict(bw=256, blocks=[1, 4]), rf.RF_ERR_INVALID_ARG),                 # out of range
        (dict(bw=256, blocks=[1, 2, 3]), rf.RF_ERR_INVALID_ARG),              # desc_out width differs
        (dict(bw=256, blocks=[0, 1], out=rf.gram_desc(512, 3, torch.bfloat16, d_out=512)), rf.RF_ERR_INVALID_ARG),
        (dict(bw=256, blocks=[0, 1], sout=256), rf.RF_ERR_INVALID_ARG),       # same buffer
    ]
    for kw, status in cases:
        with pytest.raises(rf.RidgeFillError) as e:
            rf.rf_gram_select(src, 256, kw["bw"], kw["blocks"], kw.get("out", ok), kw.get("sout", 512), stream=0)
        assert e.value.status == status, kw


def test_solve_pinv_validation_before_enqueue():
    desc = rf.gram_desc(256, 2, torch.float32)
    assert rf.rf_solve_pinv_workspace_bytes(desc, 2) > rf.rf_solve_workspace_bytes(desc, 2) + 256 * 256 * 8
    ws = torch.empty(16, dtype=torch.uint8)
    for lam, tol, sweeps, targets, status in [(-1.0, 1e-8, 15, [0], rf.RF_ERR_INVALID_ARG),
                                              (0.0, 1.5, 15, [0], rf.RF_ERR_INVALID_ARG),
                                              (0.0, 1e-8, 0, [0], rf.RF_ERR_INVALID_ARG),
                                              (0.0, 1e-8, 15, [2], rf.RF_ERR_INVALID_ARG),
                                              (0.0, 1e-8, 15, [0], rf.RF_ERR_WORKSPACE)]:
        with pytest.raises(rf.RidgeFillError) as e:
            rf._check(rf._lib.rf_solve_pinv(C.byref(desc), 256, lam, 0, tol, sweeps, (C.c_int32 * 1)(*targets), 1,
                                            None, None, None, 256, 16, None))
        assert e.value.status == status, (lam, tol, sweeps, targets)


def test_fill_static_refuses_oversized_requests_before_any_device_call():
    # one layer of 20000 rows at d = 4096 needs 164 MB of workspace, more than the static buffer
    assert rf.rf_fill_static_scratch_bytes() == 96 << 20
    w = _weights(d=4096, H=8, dh=128, dtype=torch.bfloat16)
    cd = rf.cache_desc(8, 128, 20000, rf.RF_LAYOUT_CONTIGUOUS, torch.bfloat16)
    X = torch.empty(20000, 4096, dtype=torch.bfloat16)
    with pytest.raises(rf.RidgeFillError) as e:
        rf.rf_fill_static(w, X, 0, 20000, 0, cd, [256], [256], None, 256, 20000, stream=0)
    assert e.value.status == rf.RF_ERR_UNSUPPORTED and "static buffer" in e.value.message
    # a request that fits is still validated first (here: no RoPE table)
    with pytest.raises(rf.RidgeFillError) as e:
        rf.rf_fill_static(w, X[:64], 0, 64, 0, cd, [256], [256], None, None, 64, stream=0)
    assert e.value.status == rf.RF_ERR_INVALID_ARG


def _cweights(d=256, H=4, dh=64, n=1, ptr=256, c_v=None):
    c_v = [ptr] * n if c_v is None else c_v
    return rf.ComposedFillWeights(d, H, dh, 1e-6, [ptr] * n, [ptr] * n, [ptr] * n, [ptr] * n, [ptr] * n, c_v)


def test_fill_compose_validation_before_enqueue():
    bf = torch.bfloat16
    w = _weights(dtype=bf)
    # one layer slot: W^T [d][d] bf16, then [W_kv diag(gamma)] as [hi | lo], [2 kvw][2d] bf16 (d = kvw = 256)
    assert rf.rf_fill_compose_workspace_bytes(w) == 2 * 256 * 256 + 8 * 256 * 256
    ws = _aligned_bytes(rf.rf_fill_compose_workspace_bytes(w))
    cases = [
        (dict(w=_weights(dtype=torch.float32)), rf.RF_ERR_UNSUPPORTED),           # BF16 only
        (dict(w=_weights(d=320, dtype=bf)), rf.RF_ERR_UNSUPPORTED),
        (dict(w=_weights(dh=96, H=8, dtype=bf)), rf.RF_ERR_UNSUPPORTED),
        (dict(w=_weights(H=1, dh=64, dtype=bf)), rf.RF_ERR_UNSUPPORTED),        # kv width 64, not a tile
        (dict(out=_cweights(ptr=264)), rf.RF_ERR_INVALID_ARG),                     # outputs 8-byte aligned
        (dict(out=_cweights(ptr=0)), rf.RF_ERR_INVALID_ARG),                       # null outputs
        (dict(ws=_aligned_bytes(256)), rf.RF_ERR_WORKSPACE),
        (dict(ws=_aligned_bytes(len(ws) + 512)[8:]), rf.RF_ERR_INVALID_ARG),      # misaligned workspace
        (dict(w=_weights_q8(dtype=bf)), rf.RF_ERR_UNSUPPORTED),                   # int8 maps are not composed
    ]
    for kw, status in cases:
        args = dict(w=w, out=_cweights(), ws=ws)
        args.update(kw)
        with pytest.raises(rf.RidgeFillError) as e:
            rf.rf_fill_compose(args["w"], args["out"], args["ws"], stream=0)
        assert e.value.status == status, kw
    rf.rf_fill_compose(w, _cweights(), ws, stream=0, n_layers=0)   # no layers: nothing to do


def test_fill_composed_validation_before_enqueue():
    bf = torch.bfloat16
    cache = rf.cache_desc(4, 64, 512, rf.RF_LAYOUT_CONTIGUOUS, bf)
    X = torch.empty(512, 256, dtype=bf)
    rope = torch.empty(512, 64)
    w = _cweights()
    need = rf.rf_fill_composed_workspace_bytes(w, 512)
    assert need >= 512 * (256 // 256) * 4
    ws = _aligned_bytes(need)

    def call(w=w, t0=0, t1=512, pos0=0, cache_=cache, ws_=ws, n_layers=None):
        rf.rf_fill_composed(w, X, t0, t1, pos0, cache_, [256], [256], None, rope, 512, ws_, stream=0,
                            n_layers=n_layers)

    cases = [
        (dict(t0=5, t1=4), rf.RF_ERR_INVALID_ARG),
        (dict(w=_cweights(d=320)), rf.RF_ERR_UNSUPPORTED),
        (dict(w=_cweights(dh=96, H=8)), rf.RF_ERR_UNSUPPORTED),
        (dict(t1=513), rf.RF_ERR_INVALID_ARG),
        (dict(pos0=1), rf.RF_ERR_INVALID_ARG),                                    # rope table too short
        (dict(w=_cweights(c_v=[0])), rf.RF_ERR_INVALID_ARG),                       # null value intercepts
        (dict(ws_=_aligned_bytes(256)), rf.RF_ERR_WORKSPACE),
        (dict(cache_=rf.cache_desc(4, 64, 512, rf.RF_LAYOUT_PAGED, bf)), rf.RF_ERR_INVALID_ARG),  # no table
    ]
    for kw, status in cases:
        with pytest.raises(rf.RidgeFillError) as e:
            call(**kw)
        assert e.value.status == status, kw
    call(t0=7, t1=7)          # empty range: nothing to do
    call(n_layers=0)          # no layers: nothing to do


def test_gdn_state_validation_before_enqueue():
    P = C.POINTER(C.c_void_p)

    def call(n_heads=4, d_k=128, d_v=128, dtype=rf.RF_BF16, normalise=1, eps=1e-6, n_layers=1, ld_k=None,
             ld_v=None, n_tokens=16, state=256):
        desc = rf.rf_gdn_desc(n_heads, d_k, d_v, dtype, normalise, eps)
        ptrs = (C.c_void_p * 64)(*([256] * 64))
        states = (C.c_void_p * 64)(*([state] * 64))
        rf._check(rf._lib.rf_gdn_state(C.byref(desc), n_layers, ptrs, ptrs, n_heads * d_k if ld_k is None else ld_k,
                                       n_heads * d_v if ld_v is None else ld_v, C.cast(ptrs, P), C.cast(ptrs, P),
                                       n_tokens, C.cast(states, P), None))

    cases = [
        (dict(d_k=96), rf.RF_ERR_UNSUPPORTED),
        (dict(n_layers=65), rf.RF_ERR_UNSUPPORTED),
        (dict(n_layers=-1), rf.RF_ERR_INVALID_ARG),
        (dict(d_v=4097), rf.RF_ERR_INVALID_ARG),
        (dict(n_heads=0), rf.RF_ERR_INVALID_ARG),
        (dict(dtype=7), rf.RF_ERR_INVALID_ARG),
        (dict(normalise=2), rf.RF_ERR_INVALID_ARG),
        (dict(eps=-1.0), rf.RF_ERR_INVALID_ARG),
        (dict(ld_k=4 * 128 - 8), rf.RF_ERR_INVALID_ARG),                           # rows shorter than the heads
        (dict(ld_v=4 * 128 - 8), rf.RF_ERR_INVALID_ARG),
        (dict(state=264), rf.RF_ERR_INVALID_ARG),                                  # states 8-byte aligned
        (dict(state=0), rf.RF_ERR_INVALID_ARG),
    ]
    for kw, status in cases:
        with pytest.raises(rf.RidgeFillError) as e:
            call(**kw)
        assert e.value.status == status, kw
    call(n_tokens=0)          # no tokens: nothing to do
    call(n_layers=0)          # no layers: nothing to do


def test_solve_headwise_validation_before_enqueue():
    # head_dim must divide the targets' width and d must be whole source layers of that width
    desc = rf.gram_desc(512, 1, torch.bfloat16, d_out=256)
    ws = _aligned_bytes(rf.rf_solve_workspace_bytes(desc, 1, 1))
    info = torch.zeros(1, dtype=torch.int32)
    for hd in (0, -8, 12, 96, 512):
        with pytest.raises(rf.RidgeFillError) as e:
            rf.rf_solve_headwise(desc, 256, 0.1, 0, hd, [0], None, None, None, info, ws, stream=0)
        assert e.value.status == rf.RF_ERR_INVALID_ARG, hd
    odd = rf.gram_desc(768, 1, torch.bfloat16, d_out=512)     # 768 is not a multiple of 512
    with pytest.raises(rf.RidgeFillError) as e:
        rf.rf_solve_headwise(odd, 256, 0.1, 0, 128, [0], None, None, None, info, ws, stream=0)
    assert e.value.status == rf.RF_ERR_INVALID_ARG
    with pytest.raises(rf.RidgeFillError) as e:              # then the rf_solve checks: lambda
        rf.rf_solve_headwise(desc, 256, -1.0, 0, 128, [0], None, None, None, info, ws, stream=0)
    assert e.value.status == rf.RF_ERR_INVALID_ARG
