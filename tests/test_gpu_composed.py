"""The composed fill (rf_fill_compose + rf_fill_composed) against the oracle: every filled row
at small sizes (ragged ranges, several tiles, both head widths, paged, per-head key norm) and
sampled rows at the workloads' full sizes in the launch configuration the benchmark uses.
The composed weights themselves are checked against their definitions on the unpacked maps."""
import numpy as np
import pytest
import torch

import synth
from gpu_cases import FillCase, f64, log, run_fill_case
from test_gpu_fill import SMALL_BF16, SMALL_BF16_H64, SMALL_PAGED
from test_gpu_fullsize import _boundary_sample
from test_gpu_pack import unpack

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _check(res, label):
    log(f"[composed] {label}: max_err={res['max_err']:.3e} tol={res['tol']} k={np.round(res['k_err'], 5)} "
        f"v={np.round(res['v_err'], 5)} sentinels={res['sentinel_ok']} finite={res['finite']}")
    assert res["finite"] and res["sentinel_ok"] and res["max_err"] <= res["tol"], label


def test_composed_weights_match_their_definitions():
    # T = strict upper(2 W^T W), q = [2 W^T b, diag(W^T W), |b|^2], M = W_kv diag(gamma) W and
    # c = W_kv diag(gamma) b, from the bf16 weights as stored (fp64 on the host)
    from linear_kv_cache_amd.runner import compose_weights, fill_weights
    cfg = SMALL_BF16
    layers = cfg.filled_layers[:2]
    ws = [synth.layer_weights(cfg, l, device="cuda") for l in layers]
    fw = fill_weights(cfg.d, cfg.n_kv_heads, cfg.head_dim, cfg.rms_eps, cfg.torch_dtype, [w.W_map for w in ws],
                      [w.b_map for w in ws], [w.gamma for w in ws], [w.W_k for w in ws], [w.W_v for w in ws])
    cw = compose_weights(fw)
    torch.cuda.synchronize()
    d, kvw, hd = cfg.d, cfg.n_kv_heads * cfg.head_dim, cfg.head_dim
    for li, w in enumerate(ws):
        W, b, g = f64(w.W_map), f64(w.b_map), f64(w.gamma)
        G = W.T @ W
        T_ref = np.triu(2 * G, 1)
        T = unpack(cw.T[li], d, d).astype(np.int16)
        T = torch.from_numpy(T).view(torch.bfloat16).double().numpy()
        # blocks below the 256 x 256 block diagonal are never read
        blk = np.kron(np.triu(np.ones((d // 256, d // 256))), np.ones((256, 256))).astype(bool)
        e_T = np.max(np.abs(T - T_ref)[blk]) / np.max(np.abs(T_ref))
        q = f64(cw.q[li])
        e_q = max(np.max(np.abs(q[:d] - 2 * W.T @ b)) / np.max(np.abs(2 * W.T @ b)),
                  np.max(np.abs(q[d:2 * d] - np.diag(G))) / np.max(np.diag(G)), abs(q[2 * d] - b @ b) / (b @ b))
        errs = []
        for Wkv, M, c in ((w.W_k, cw.M_k[li], cw.c_k[li]), (w.W_v, cw.M_v[li], cw.c_v[li])):
            A = f64(Wkv)
            M_ref = (A * g[None, :]) @ W
            Mg = torch.from_numpy(unpack(M, kvw, d, hd).astype(np.int16)).view(torch.bfloat16).double().numpy()
            errs.append(np.max(np.abs(Mg - M_ref)) / np.max(np.abs(M_ref)))
            c_ref = (A * g[None, :]) @ b
            errs.append(np.max(np.abs(f64(c) - c_ref)) / np.max(np.abs(c_ref)))
        log(f"[composed] layer {li}: T {e_T:.2e} q {e_q:.2e} M, c {np.round(errs, 7).tolist()}")
        # bf16 storage of T and M: half an ulp (2^-9) of the largest entry at most
        assert e_T <= 2 ** -8 and max(errs[0], errs[2]) <= 2 ** -8
        assert e_q <= 1e-6 and max(errs[1], errs[3]) <= 1e-6


def test_composed_fill_bf16_ragged_offset_range():
    _check(run_fill_case(FillCase(SMALL_BF16, 37, 737, pos0=11, composed=True)), "d512 x3 [37,737)")


def test_composed_fill_head_dim_64_and_identity_maps():
    _check(run_fill_case(FillCase(SMALL_BF16_H64, 0, 600, composed=True)), "d256 dh64 [0,600)")
    _check(run_fill_case(FillCase(SMALL_BF16_H64, 3, 259, maps="identity", composed=True)), "d256 dh64 identity")


def test_composed_fill_paged_chunked_unaligned():
    _check(run_fill_case(FillCase(SMALL_PAGED, 19, 1100, chunk=300, composed=True)), "paged d512 chunks of 300")


def test_composed_fill_per_head_key_norm():
    _check(run_fill_case(FillCase(SMALL_BF16, 5, 700, pos0=3, k_norm=True, composed=True)), "d512 key norm")


def test_composed_fill_single_token_and_tile_edges():
    for t0, t1 in ((0, 1), (255, 257), (511, 513)):
        _check(run_fill_case(FillCase(SMALL_BF16, t0, t1, composed=True)), f"d512 [{t0},{t1})")


def test_composed_fill_deterministic_and_empty_ranges():
    # the composition and the composed fill are bitwise deterministic (fixed-order reductions,
    # no atomics), and an empty token range writes nothing
    from linear_kv_cache_amd.runner import ComposedFiller, alloc_cache, fill_weights
    cfg = SMALL_BF16
    ws = [synth.layer_weights(cfg, l, device="cuda") for l in cfg.filled_layers[:2]]
    fw = fill_weights(cfg.d, cfg.n_kv_heads, cfg.head_dim, cfg.rms_eps, cfg.torch_dtype, [w.W_map for w in ws],
                      [w.b_map for w in ws], [w.gamma for w in ws], [w.W_k for w in ws], [w.W_v for w in ws])
    X = synth.hidden_states(cfg, 700, "prompt", device="cuda")
    outs = []
    for _ in range(2):
        cache = alloc_cache(2, cfg.n_kv_heads, cfg.head_dim, 700, cfg.torch_dtype, "cuda", sentinel=3.0)
        filler = ComposedFiller(fw, cfg.rope_base, 700, 700, "cuda")
        for t in (0, 350, 700):
            filler.fill(X, t, t, 0, cache)
        torch.cuda.synchronize()
        assert all(bool(torch.all(t == 3.0)) for t in cache.k + cache.v)
        filler.fill(X, 0, 700, 0, cache)
        outs.append(torch.cat(cache.k + cache.v))
    torch.cuda.synchronize()
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))


@pytest.mark.slow
@pytest.mark.timeout(300)
def test_composed_fill_llama8b_shaped_full():
    cfg = synth.C2
    sample = _boundary_sample(0, cfg.fill_t1, cfg.fill_chunk, 31)
    _check(run_fill_case(FillCase(cfg, 0, cfg.fill_t1, maps="law", sample=sample, gen_device="cuda", composed=True)),
           "d4096 x16 layers T16384")


@pytest.mark.slow
@pytest.mark.timeout(300)
def test_composed_fill_27b_shaped_full():
    cfg = synth.C3
    sample = _boundary_sample(cfg.fill_t0, cfg.fill_t1, cfg.fill_chunk, 32)
    _check(run_fill_case(FillCase(cfg, cfg.fill_t0, cfg.fill_t1, sample=sample, gen_device="cuda",
                                  max_tokens=cfg.prompt_tokens, composed=True)), "d5120 x48 layers [2048,28672)")


@pytest.mark.slow
@pytest.mark.timeout(300)
def test_composed_fill_long_context_paged_chunks():
    cfg = synth.C5
    sample = _boundary_sample(0, cfg.fill_t1, cfg.fill_chunk, 33)
    _check(run_fill_case(FillCase(cfg, 0, cfg.fill_t1, chunk=cfg.fill_chunk, sample=sample, gen_device="cuda",
                                  max_tokens=cfg.prompt_tokens, composed=True)), "d4096 x16 layers paged T131072")
