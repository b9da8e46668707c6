"""rf_fill_static (the fill with the library's static scratch buffer, for callers that cannot
allocate) against rf_fill on the same inputs: bit-identical caches on two calls in a row, the
second smaller than the first, so the second call runs on a buffer that holds the first
call's contents."""
import pytest
import torch

import synth
from gpu_cases import log

pytestmark = pytest.mark.gpu

BF16 = synth.scaled(synth.C2, name="bf16-d512", d=512, n_layers=5, split=2, n_kv_heads=2, head_dim=128,
                    prompt_tokens=1400)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _equal(a, b):
    view = torch.int16 if a.dtype == torch.bfloat16 else torch.int32
    return torch.equal(a.view(view), b.view(view))


@pytest.mark.parametrize("cfg", [BF16, synth.C1], ids=["bf16", "fp32"])
def test_fill_static_matches_fill_on_two_calls(cfg):
    import linear_kv_cache_amd as rf
    from linear_kv_cache_amd.runner import Filler, alloc_cache, fill_weights
    layers = cfg.filled_layers
    ws = [synth.layer_weights(cfg, l, device="cuda") for l in layers]
    fw = fill_weights(cfg.d, cfg.n_kv_heads, cfg.head_dim, cfg.rms_eps, cfg.torch_dtype, [w.W_map for w in ws],
                      [w.b_map for w in ws], [w.gamma for w in ws], [w.W_k for w in ws], [w.W_v for w in ws])
    T = max(1400, cfg.prompt_tokens)
    for call, (t0, t1, pos0) in enumerate(((5, 1300, 3), (40, 337, 0))):
        X = synth.hidden_states(cfg, t1 - t0, "prompt", chunk=call, device="cuda")
        filler = Filler(fw, cfg.rope_base, T + 8, t1 - t0, "cuda")
        caches = []
        for static in (False, True):
            cache = alloc_cache(len(layers), cfg.n_kv_heads, cfg.head_dim, T, cfg.torch_dtype, "cuda")
            if static:
                rf.rf_fill_static(fw, X, t0, t1, pos0, cache.desc, cache.k, cache.v, None, filler.rope,
                                  filler.rope_len)
            else:
                filler.fill(X, t0, t1, pos0, cache)
            caches.append(cache)
        torch.cuda.synchronize()
        for li in range(len(layers)):
            assert _equal(caches[0].k[li], caches[1].k[li]) and _equal(caches[0].v[li], caches[1].v[li]), (call, li)
        log(f"[no-alloc] {cfg.name} call {call} rows [{t0}, {t1}): rf_fill_static equals rf_fill bit for bit")
