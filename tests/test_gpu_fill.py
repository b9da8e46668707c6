"""GPU parity of rf_fill against the oracle (element by element at sizes the oracle finishes in
seconds; sampled rows at full size).  Every case checks the untouched-row contract too."""
import numpy as np
import pytest
import torch

import synth
from gpu_cases import FillCase, log, run_fill_case

pytestmark = pytest.mark.gpu

SMALL_BF16 = synth.scaled(synth.C2, name="bf16-d512", d=512, n_layers=5, split=2, n_kv_heads=2, head_dim=128,
                          prompt_tokens=900)
SMALL_BF16_H64 = synth.scaled(synth.C2, name="bf16-d256-dh64", d=256, n_layers=3, split=1, n_kv_heads=4,
                              head_dim=64, prompt_tokens=600, rope_base=1e4)
SMALL_PAGED = synth.scaled(synth.C5, name="paged-d512", d=512, n_layers=4, split=1, n_kv_heads=2, head_dim=128,
                           prompt_tokens=1200)
# K/V widths that are whole 512-feature tiles run the K/V product on 512 x 128 tiles (the
# configs above, 256 wide, the 256 x 256 kernel): 4 x 128 and 8 x 64 heads
WIDE_BF16 = synth.scaled(synth.C2, name="bf16-d512-kv512", d=512, n_layers=4, split=2, n_kv_heads=4, head_dim=128,
                         prompt_tokens=900)
WIDE_BF16_H64 = synth.scaled(synth.C2, name="bf16-d512-kv8x64", d=512, n_layers=3, split=1, n_kv_heads=8,
                             head_dim=64, prompt_tokens=600, rope_base=1e4)
# (the Llama-8B-shaped input law, paged: at d = 512 the long-context law's five 20x outlier
# channels make K heavy-tailed enough that bf16 storage alone reaches 2.2e-2 of RMS, with the
# 256 x 256 kernel and this one alike)
WIDE_PAGED = synth.scaled(synth.C2, name="paged-d512-kv1024", d=512, n_layers=3, split=1, n_kv_heads=8,
                          head_dim=128, prompt_tokens=1200, paged=True, block_size=16)


def _check(res, label):
    log(f"[fill] {label}: max_err={res['max_err']:.3e} tol={res['tol']} k={np.round(res['k_err'], 5)} "
        f"v={np.round(res['v_err'], 5)} sentinels={res['sentinel_ok']} finite={res['finite']}")
    assert res["finite"], label
    assert res["sentinel_ok"], label
    assert res["max_err"] <= res["tol"], label


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_fill_tiny_fp32_all_rows():
    # d=256, 4 filled layers, 4 KV heads x 64, fp32 storage, T=512
    _check(run_fill_case(FillCase(synth.C1, 0, 512)), "C1 fp32")


def test_fill_bf16_ragged_offset_range():
    # 3 filled layers, rows [37, 737): two full 256-token tiles and a ragged tail, pos0 = 5
    _check(run_fill_case(FillCase(SMALL_BF16, 37, 737, pos0=5)), "bf16 d512 ragged")


def test_fill_bf16_head_dim_64_and_identity_maps():
    _check(run_fill_case(FillCase(SMALL_BF16_H64, 3, 517, maps="identity")), "bf16 dh64 identity")
    _check(run_fill_case(FillCase(SMALL_BF16_H64, 0, 600, maps="random", pos0=70000)), "bf16 dh64 far pos")


def test_fill_paged_chunked_unaligned():
    # paged cache (block 16, shuffled table), fill [19, 1100) in chunks of 300 tokens
    _check(run_fill_case(FillCase(SMALL_PAGED, 19, 1100, chunk=300)), "paged chunked")


@pytest.mark.parametrize("composed", [False, True])
def test_fill_512_wide_kv_tiles(composed):
    # ragged range across several 128-token tiles, far positions, identity maps, paged in
    # chunks, both head widths, per-head key norm.  Each case keeps a side of a layer under
    # about 0.7 M values: the bar is a maximum over every value, and the bf16 rounding of the
    # stored cache alone (half an ulp, up to 2^-8 of a value) reaches it for the largest values
    # of a few million Gaussian draws (about 5.4 RMS)
    for case, label in ((FillCase(WIDE_BF16, 37, 737, pos0=5, composed=composed), "kv512 ragged"),
                        (FillCase(WIDE_BF16, 0, 129, composed=composed), "kv512 [0,129)"),
                        (FillCase(WIDE_BF16, 5, 700, pos0=70000, k_norm=True, composed=composed), "kv512 key norm"),
                        (FillCase(WIDE_BF16_H64, 3, 517, maps="identity", composed=composed), "kv8x64 identity"),
                        (FillCase(WIDE_BF16_H64, 0, 600, k_norm=True, composed=composed), "kv8x64 key norm"),
                        (FillCase(WIDE_PAGED, 19, 619, chunk=200, composed=composed), "kv1024 paged chunks"),
                        (FillCase(WIDE_PAGED, 0, 600, chunk=250, k_norm=True, composed=composed), "kv1024 paged key norm")):
        _check(run_fill_case(case), f"{label}{' composed' if composed else ''}")


def test_fill_per_head_key_norm():
    # keys normalised per head before the rotation (head_dim 128: the head spans two waves of a
    # tile; 64: one wave), bf16 and fp32
    _check(run_fill_case(FillCase(SMALL_BF16, 37, 737, pos0=5, k_norm=True)), "bf16 dh128 key norm")
    _check(run_fill_case(FillCase(SMALL_BF16_H64, 3, 517, maps="random", k_norm=True)), "bf16 dh64 key norm")
    _check(run_fill_case(FillCase(synth.C1, 0, 512, k_norm=True)), "C1 fp32 key norm")
    _check(run_fill_case(FillCase(SMALL_PAGED, 19, 1100, chunk=300, k_norm=True)), "paged key norm")


def test_fill_single_token_and_tile_edges():
    for t0, t1 in [(5, 6), (0, 256), (255, 257), (511, 769)]:
        _check(run_fill_case(FillCase(SMALL_BF16, t0, t1, n_layers=1)), f"rows [{t0},{t1})")


def test_empty_calls_change_nothing():
    # an empty token range (t0 == t1, at the start, inside and at the end of the prompt) and a
    # zero-row calibration chunk are no-ops: sentinel caches and an accumulated state keep every byte
    from linear_kv_cache_amd.runner import Filler, GramState, alloc_cache, fill_weights
    cfg = SMALL_BF16
    ws = [synth.layer_weights(cfg, l, device="cuda") for l in cfg.filled_layers[:2]]
    fw = fill_weights(cfg.d, cfg.n_kv_heads, cfg.head_dim, cfg.rms_eps, cfg.torch_dtype, [w.W_map for w in ws],
                      [w.b_map for w in ws], [w.gamma for w in ws], [w.W_k for w in ws], [w.W_v for w in ws])
    X = synth.hidden_states(cfg, 300, "prompt", device="cuda")
    cache = alloc_cache(2, cfg.n_kv_heads, cfg.head_dim, 300, cfg.torch_dtype, "cuda", sentinel=3.0)
    filler = Filler(fw, cfg.rope_base, 300, 300, "cuda")
    for t in (0, 17, 300):
        filler.fill(X, t, t, 0, cache)
    st = GramState(cfg.d, 2, cfg.torch_dtype, "cuda")
    Ys = [synth.late_layer_inputs(cfg, X, cfg.split + l) for l in range(2)]
    st.accumulate(X, Ys)
    before = st.buf.clone()
    st.accumulate(X[:0], [Y[:0] for Y in Ys])
    torch.cuda.synchronize()
    assert all(bool(torch.all(t == 3.0)) for t in cache.k + cache.v)
    assert torch.equal(st.buf, before) and int(st.n().item()) == 300


def test_fill_is_deterministic():
    from linear_kv_cache_amd.runner import Filler, alloc_cache, fill_weights
    cfg = SMALL_BF16
    ws = [synth.layer_weights(cfg, l, device="cuda") for l in cfg.filled_layers[:2]]
    fw = fill_weights(cfg.d, cfg.n_kv_heads, cfg.head_dim, cfg.rms_eps, cfg.torch_dtype, [w.W_map for w in ws],
                      [w.b_map for w in ws], [w.gamma for w in ws], [w.W_k for w in ws], [w.W_v for w in ws])
    X = synth.hidden_states(cfg, 700, "prompt", device="cuda")
    outs = []
    for _ in range(2):
        cache = alloc_cache(2, cfg.n_kv_heads, cfg.head_dim, 700, cfg.torch_dtype, "cuda")
        Filler(fw, cfg.rope_base, 700, 700, "cuda").fill(X, 0, 700, 0, cache)
        outs.append(torch.cat(cache.k + cache.v))
    torch.cuda.synchronize()
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))


def test_fill_streamed_maps_match_resident():
    # maps in page-locked host memory streamed through a device ring: the same kernels on the
    # same data, so the caches equal the resident fill's bit for bit; checked against the
    # oracle too.  Ring reuse (3 chunks in 2 slots), one slot (copies wait for each fill),
    # chunks of 2 layers; bf16 packed and fp32 maps; paged and contiguous
    from linear_kv_cache_amd.runner import (Filler, StreamedFiller, alloc_cache, fill_weights, gather_rows,
                                            pinned_copy)
    import oracle
    from gpu_cases import f64
    for cfg, t0, t1, slots, per, paged in [(SMALL_BF16, 37, 737, 2, 1, False), (synth.C1, 0, 512, 1, 3, False),
                                           (SMALL_PAGED, 19, 1100, 2, 2, True)]:
        layers = cfg.filled_layers
        ws = [synth.layer_weights(cfg, l, device="cuda") for l in layers]
        fw = fill_weights(cfg.d, cfg.n_kv_heads, cfg.head_dim, cfg.rms_eps, cfg.torch_dtype, [w.W_map for w in ws],
                          [w.b_map for w in ws], [w.gamma for w in ws], [w.W_k for w in ws], [w.W_v for w in ws])
        host = [pinned_copy(W.cpu()) for W in fw.W_map]
        fs = fill_weights(cfg.d, cfg.n_kv_heads, cfg.head_dim, cfg.rms_eps, cfg.torch_dtype, [w.W_map for w in ws],
                          [w.b_map for w in ws], [w.gamma for w in ws], [w.W_k for w in ws], [w.W_v for w in ws])
        fs.W_map = host
        T = max(t1, cfg.prompt_tokens)
        X = synth.hidden_states(cfg, t1 - t0, "prompt", device="cuda")
        table = synth.block_table(cfg, T, device="cuda") if paged else None
        nb = int(table.max()) + 1 if paged else None
        outs = []
        for filler in (Filler(fw, cfg.rope_base, T, t1 - t0, "cuda"),
                       StreamedFiller(fs, cfg.rope_base, T, t1 - t0, "cuda", ring_slots=slots, layers_per_slot=per)):
            cache = alloc_cache(len(layers), cfg.n_kv_heads, cfg.head_dim, T, cfg.torch_dtype, "cuda", paged=paged,
                                block_size=cfg.block_size, block_table=table, n_blocks=nb)
            filler.fill(X, t0, t1, 0, cache)
            torch.cuda.synchronize()
            outs.append(cache)
        for li in range(len(layers)):
            for a, b in ((outs[0].k[li], outs[1].k[li]), (outs[0].v[li], outs[1].v[li])):
                assert torch.equal(a.view(torch.int16 if a.dtype == torch.bfloat16 else torch.int32),
                                   b.view(torch.int16 if b.dtype == torch.bfloat16 else torch.int32)), (cfg.name, li)
        rows = np.arange(t0, t1)
        errs = []
        for li, w in enumerate(ws):
            K_ref, V_ref = oracle.fill_layer(f64(X), f64(w.W_map).T, f64(w.b_map), f64(w.gamma), f64(w.W_k).T,
                                             f64(w.W_v).T, rows.astype(np.float64), cfg.n_kv_heads, cfg.head_dim,
                                             cfg.rms_eps, cfg.rope_base)
            K = f64(gather_rows(outs[1], outs[1].k[li], t0, t1))
            V = f64(gather_rows(outs[1], outs[1].v[li], t0, t1))
            errs.append(max(float(np.max(np.abs(K - K_ref)) / np.sqrt(np.mean(K_ref ** 2))),
                            float(np.max(np.abs(V - V_ref)) / np.sqrt(np.mean(V_ref ** 2)))))
        tol = 1e-4 if cfg.dtype == "f32" else 2e-2
        log(f"[fill] streamed {cfg.name} slots={slots} per_slot={per}: bit-identical to resident, max_err={max(errs):.3e}")
        assert max(errs) <= tol


def test_fill_streamed_back_to_back_chunks():
    # a long prompt filled in token chunks, one streamed call per chunk on one stream with no
    # host synchronisation between the calls: each call's first map copies into the ring must
    # wait for the previous call's fills, so the caches still equal the resident fill's bit for bit
    from linear_kv_cache_amd.runner import Filler, StreamedFiller, alloc_cache, fill_weights, pinned_copy
    cfg = SMALL_BF16
    layers = cfg.filled_layers
    ws = [synth.layer_weights(cfg, l, device="cuda") for l in layers]
    args = (cfg.d, cfg.n_kv_heads, cfg.head_dim, cfg.rms_eps, cfg.torch_dtype, [w.W_map for w in ws],
            [w.b_map for w in ws], [w.gamma for w in ws], [w.W_k for w in ws], [w.W_v for w in ws])
    fw = fill_weights(*args)
    fs = fill_weights(*args)
    fs.W_map = [pinned_copy(W.cpu()) for W in fw.W_map]
    t0, t1, chunk = 5, 1301, 256
    X = synth.hidden_states(cfg, t1 - t0, "prompt", device="cuda")
    outs = []
    for streamed in (False, True):
        cache = alloc_cache(len(layers), cfg.n_kv_heads, cfg.head_dim, t1, cfg.torch_dtype, "cuda")
        if streamed:
            filler = StreamedFiller(fs, cfg.rope_base, t1, chunk, "cuda", ring_slots=2, layers_per_slot=1)
        else:
            filler = Filler(fw, cfg.rope_base, t1, t1 - t0, "cuda")
        torch.cuda.synchronize()
        if streamed:
            for c0 in range(t0, t1, chunk):
                c1 = min(t1, c0 + chunk)
                filler.fill(X[c0 - t0:c1 - t0], c0, c1, 0, cache)
        else:
            filler.fill(X, t0, t1, 0, cache)
        torch.cuda.synchronize()
        outs.append(cache)
    for li in range(len(layers)):
        for a, b in ((outs[0].k[li], outs[1].k[li]), (outs[0].v[li], outs[1].v[li])):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), li
    log(f"[fill] streamed back-to-back chunks of {chunk}: bit-identical to the resident fill")


def test_fill_streamed_long_prompt_in_steps():
    # one streamed call over a long range, filled in steps of 256 tokens inside each layer chunk
    # (each map copied once), paged: the caches equal the resident fill's bit for bit
    from linear_kv_cache_amd.runner import Filler, StreamedFiller, alloc_cache, fill_weights, pinned_copy
    cfg = SMALL_PAGED
    layers = cfg.filled_layers
    ws = [synth.layer_weights(cfg, l, device="cuda") for l in layers]
    args = (cfg.d, cfg.n_kv_heads, cfg.head_dim, cfg.rms_eps, cfg.torch_dtype, [w.W_map for w in ws],
            [w.b_map for w in ws], [w.gamma for w in ws], [w.W_k for w in ws], [w.W_v for w in ws])
    fw = fill_weights(*args)
    fs = fill_weights(*args)
    fs.W_map = [pinned_copy(W.cpu()) for W in fw.W_map]
    t0, t1 = 19, 1100
    T = cfg.prompt_tokens
    X = synth.hidden_states(cfg, t1 - t0, "prompt", device="cuda")
    table = synth.block_table(cfg, T, device="cuda")
    nb = int(table.max()) + 1
    outs = []
    for filler in (Filler(fw, cfg.rope_base, T, t1 - t0, "cuda"),
                   StreamedFiller(fs, cfg.rope_base, T, t1 - t0, "cuda", ring_slots=2, layers_per_slot=1,
                                  rows_per_fill=256)):
        cache = alloc_cache(len(layers), cfg.n_kv_heads, cfg.head_dim, T, cfg.torch_dtype, "cuda", paged=True,
                            block_size=cfg.block_size, block_table=table, n_blocks=nb)
        filler.fill(X, t0, t1, 0, cache)
        torch.cuda.synchronize()
        outs.append(cache)
    for li in range(len(layers)):
        for a, b in ((outs[0].k[li], outs[1].k[li]), (outs[0].v[li], outs[1].v[li])):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), li
    log("[fill] streamed in steps of 256 tokens: bit-identical to the resident fill")


def test_fill_without_rope_table_builds_it_in_the_workspace():
    # d_rope NULL: the library builds the table of the call's positions at the end of the
    # workspace (from the weights' rope_base, the same fp64 angles) and the caches equal those
    # of the caller's table bit for bit: rf_fill on both K/V kernels, rf_fill_static,
    # rf_fill_composed and rf_fill_streamed in token steps, at t0 > 0 and pos0 > 0
    import dataclasses

    import linear_kv_cache_amd as rf
    from linear_kv_cache_amd.runner import (ComposedFiller, Filler, StreamedFiller, alloc_cache, device_bytes,
                                            fill_weights, pinned_copy)
    for cfg in (SMALL_BF16, WIDE_BF16):
        t0, t1, pos0 = 37, 737, 1234
        layers = cfg.filled_layers
        ws_ = [synth.layer_weights(cfg, l, device="cuda") for l in layers]
        fw = fill_weights(cfg.d, cfg.n_kv_heads, cfg.head_dim, cfg.rms_eps, cfg.torch_dtype, [w.W_map for w in ws_],
                          [w.b_map for w in ws_], [w.gamma for w in ws_], [w.W_k for w in ws_], [w.W_v for w in ws_])
        fw.rope_base = cfg.rope_base
        T = max(t1, cfg.prompt_tokens)
        X = synth.hidden_states(cfg, t1 - t0, "prompt", device="cuda")
        rope_extra = rf.rf_rope_workspace_bytes(cfg.head_dim, t1 - t0)
        pairs = []
        # rf_fill
        f = Filler(fw, cfg.rope_base, pos0 + T, t1 - t0, "cuda")
        wsn = device_bytes(f.ws.numel() + rope_extra, "cuda")
        for rope in (f.rope, None):
            c = alloc_cache(len(layers), cfg.n_kv_heads, cfg.head_dim, T, cfg.torch_dtype, "cuda")
            rf.rf_fill(fw, X, t0, t1, pos0, c.desc, c.k, c.v, None, rope, f.rope_len, f.ws if rope is not None else wsn)
            pairs.append(("rf_fill", c))
        # rf_fill_static
        for rope in (f.rope, None):
            c = alloc_cache(len(layers), cfg.n_kv_heads, cfg.head_dim, T, cfg.torch_dtype, "cuda")
            rf.rf_fill_static(fw, X, t0, t1, pos0, c.desc, c.k, c.v, None, rope, f.rope_len)
            pairs.append(("rf_fill_static", c))
        # rf_fill_composed
        cf = ComposedFiller(fw, cfg.rope_base, pos0 + T, t1 - t0, "cuda")
        wsc = device_bytes(cf.ws.numel() + rope_extra, "cuda")
        for rope in (cf.rope, None):
            c = alloc_cache(len(layers), cfg.n_kv_heads, cfg.head_dim, T, cfg.torch_dtype, "cuda")
            rf.rf_fill_composed(cf.w, X, t0, t1, pos0, c.desc, c.k, c.v, None, rope, cf.rope_len,
                                cf.ws if rope is not None else wsc)
            pairs.append(("rf_fill_composed", c))
        # rf_fill_streamed in steps of 256 tokens
        sw = dataclasses.replace(fw, W_map=[pinned_copy(W.cpu()) for W in fw.W_map])
        sf = StreamedFiller(sw, cfg.rope_base, pos0 + T, t1 - t0, "cuda", ring_slots=2, layers_per_slot=1,
                            rows_per_fill=256)
        wss = device_bytes(sf.ws.numel() + rope_extra, "cuda")
        for rope in (sf.rope, None):
            c = alloc_cache(len(layers), cfg.n_kv_heads, cfg.head_dim, T, cfg.torch_dtype, "cuda")
            rf.rf_fill_streamed(sw, X, t0, t1, pos0, c.desc, c.k, c.v, None, rope, sf.rope_len,
                                sf.ws if rope is not None else wss, sf.ring, sf.ring_slots, sf.layers_per_slot,
                                torch.cuda.current_stream(), sf.copy_stream, rows_per_fill=256)
            pairs.append(("rf_fill_streamed", c))
        torch.cuda.synchronize()
        for i in range(0, len(pairs), 2):
            (name, a), (_, b) = pairs[i], pairs[i + 1]
            for li in range(len(layers)):
                for x, y in ((a.k[li], b.k[li]), (a.v[li], b.v[li])):
                    assert torch.equal(x.view(torch.int16), y.view(torch.int16)), (cfg.name, name, li)
        log(f"[fill] {cfg.name}: no rope table given -> built in the workspace, bit-identical (fill, static, "
            f"composed, streamed)")
