"""Weight-only int8 maps on the GPU.  rf_quantize_map's codes and scales equal the oracle's
quantiser bit for bit (both decide each code in fp32).  The fill with int8 maps (resident, and
streamed through the ring) matches the oracle's fill with the oracle's own codes dequantised,
on the 256 x 256 and the 512 x 128 K/V kernels.  The streamed and static fills equal the
resident int8 fill bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_cases import FillCase, f64, log, run_fill_case

pytestmark = pytest.mark.gpu

KV2 = synth.scaled(synth.C2, name="i8-d512-kv256", d=512, n_layers=4, split=2, n_kv_heads=2, head_dim=128,
                   prompt_tokens=900)
KV4 = synth.scaled(synth.C2, name="i8-d512-kv512", d=512, n_layers=4, split=2, n_kv_heads=4, head_dim=128,
                   prompt_tokens=900)
PAGED = synth.scaled(synth.C2, name="i8-paged-d768-kv1024", d=768, n_layers=3, split=1, n_kv_heads=8, head_dim=128,
                     prompt_tokens=700, paged=True, block_size=16)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _unpack(q: torch.Tensor, rows: int, cols: int) -> np.ndarray:
    """Row-major codes from the packed order (the layout rf_pack_weights documents, one byte
    per element)."""
    qn = q.cpu().numpy().reshape(-1)
    r = np.arange(rows)[:, None]
    k = np.arange(cols)[None, :]
    rt = r % 256
    idx = ((r // 256) * 256 * cols + (k // 64) * 16384 + (rt // 64) * 4096 + ((k % 64) // 16) * 1024
           + ((rt % 64) // 32) * 512 + (((k % 16) // 8) * 32 + rt % 32) * 8 + k % 8)
    return qn[idx]


def test_quantize_map_matches_oracle_bit_for_bit():
    import linear_kv_cache_amd as rf
    rng = np.random.default_rng(21)
    rows, cols, ld = 512, 320, 384
    W = (rng.standard_normal((rows, ld)) * rng.lognormal(0, 2, (rows, 1))).astype(np.float32)
    W[3] = 0.0                                                   # a zero row
    s0 = np.float32(2.0 ** -9)
    W[7, :8] = s0 * np.array([127, 2.5, 3.5, -2.5, -0.5, 0.5, 1.5, -126.5], dtype=np.float32)   # ties
    W[7, 8:] = 0.0
    W[11] = 0.0
    W[11, 200] = -3.0                                            # a single negative maximum
    W[13] = np.float32(1e-30) * rng.standard_normal(ld).astype(np.float32)   # tiny scales
    Wd = torch.from_numpy(W).cuda()
    view = Wd[:, :cols]                                          # row stride 384 > cols
    q = torch.empty(rows, cols, dtype=torch.int8, device="cuda")
    s = torch.empty(rows, dtype=torch.float32, device="cuda")
    rf.rf_quantize_map(view, q, s)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_rows(W[:, :cols])
    got = _unpack(q, rows, cols)
    assert np.array_equal(s.cpu().numpy(), s_ref)
    assert np.array_equal(got, q_ref), int(np.sum(got != q_ref))
    assert got[7, :8].tolist() == [127, 2, 4, -2, 0, 0, 2, -126]
    log(f"[quant] {rows}x{cols} (ld {ld}): codes and scales bit-identical to the oracle")


@pytest.mark.parametrize("cfg,t0,t1,chunk,pos0", [(KV2, 37, 737, None, 5), (KV4, 0, 600, 256, 70000),
                                                  (PAGED, 19, 619, 200, 0)])
def test_fill_int8_maps_against_oracle(cfg, t0, t1, chunk, pos0):
    res = run_fill_case(FillCase(cfg, t0, t1, pos0=pos0, chunk=chunk, int8_maps=True))
    log(f"[quant] fill {cfg.name} [{t0},{t1}) int8 maps: k_err={max(res['k_err']):.3e} "
        f"v_err={max(res['v_err']):.3e} (tol {res['tol']})")
    assert res["finite"] and res["sentinel_ok"]
    assert res["max_err"] <= res["tol"], res


def test_int8_streamed_and_static_equal_resident():
    import linear_kv_cache_amd as rf
    from linear_kv_cache_amd.runner import Filler, StreamedFiller, alloc_cache, fill_weights, pinned_copy
    cfg, t0, t1 = KV4, 21, 621
    layers = cfg.filled_layers
    ws = [synth.layer_weights(cfg, l, device="cuda") for l in layers]
    args = (cfg.d, cfg.n_kv_heads, cfg.head_dim, cfg.rms_eps, cfg.torch_dtype, [w.W_map for w in ws],
            [w.b_map for w in ws], [w.gamma for w in ws], [w.W_k for w in ws], [w.W_v for w in ws])
    fw = fill_weights(*args, int8_maps=True)
    fs = fill_weights(*args, int8_maps=True)
    fs.W_map = [pinned_copy(q.cpu()) for q in fs.W_map]
    T = max(t1, cfg.prompt_tokens)
    X = synth.hidden_states(cfg, t1 - t0, "prompt", device="cuda")
    caches = []
    for kind in ("resident", "streamed", "static"):
        cache = alloc_cache(len(layers), cfg.n_kv_heads, cfg.head_dim, T, cfg.torch_dtype, "cuda")
        if kind == "resident":
            Filler(fw, cfg.rope_base, T, t1 - t0, "cuda").fill(X, t0, t1, 0, cache)
        elif kind == "streamed":
            StreamedFiller(fs, cfg.rope_base, T, t1 - t0, "cuda", ring_slots=2, layers_per_slot=1).fill(X, t0, t1, 0,
                                                                                                    cache)
        else:
            f = Filler(fw, cfg.rope_base, T, t1 - t0, "cuda")
            rf.rf_fill_static(fw, X, t0, t1, 0, cache.desc, cache.k, cache.v, None, f.rope, f.rope_len)
        torch.cuda.synchronize()
        caches.append(cache)
    for kind, c in zip(("streamed", "static"), caches[1:]):
        for li in range(len(layers)):
            for a, b in ((caches[0].k[li], c.k[li]), (caches[0].v[li], c.v[li])):
                assert torch.equal(a.view(torch.int16), b.view(torch.int16)), (kind, li)
    log("[quant] int8 maps: streamed and static fills bit-identical to the resident fill")


@pytest.mark.timeout(300)
def test_fill_int8_maps_llama8b_shaped_full_sampled():
    # the benchmark's launch configuration (16 layers x 16384 tokens, d = 4096), sampled rows:
    # every 256-token tile edge and seeded random rows
    cfg = synth.C2
    rng = np.random.default_rng(31)
    edges = {0, 1, cfg.fill_t1 - 1, cfg.fill_t1 - 2}
    for b in range(256, cfg.fill_t1, 256):
        edges.update({b - 1, b})
    sample = sorted(edges | set(rng.integers(0, cfg.fill_t1, 24).tolist()))
    res = run_fill_case(FillCase(cfg, 0, cfg.fill_t1, maps="law", sample=sample, gen_device="cuda", int8_maps=True))
    log(f"[quant] full-size int8 fill: max_err={res['max_err']:.3e} (tol {res['tol']})")
    assert res["finite"] and res["sentinel_ok"]
    assert res["max_err"] <= res["tol"], res
