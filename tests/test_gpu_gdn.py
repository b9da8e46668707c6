"""The Gated DeltaNet state update on the GPU (rf_gdn_state) against the oracle's sequential
recurrence: element by element at small sizes (several token blocks and a ragged tail, ragged
value widths, both key widths, bf16 and fp32 rows, with and without key normalisation, chunked
continuation, several layers per call), and on sampled heads of a full 16384-token prompt."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_cases import f64, log

pytestmark = pytest.mark.gpu

GDN_TOL = 1e-4   # max |S - S*| / max |S*|: fp32 arithmetic over a contracting recurrence


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _run(layers, H, dk, dv, T, dtype, normalise, chunks=None, S0=None, seed=5):
    import linear_kv_cache_amd as rf
    ins = [synth.gdn_inputs(seed, l, T, H, dk, dv, dtype) for l in range(layers)]
    if not normalise:
        # keys of about unit length, so beta |k|^2 < 2 keeps the recurrence contracting
        ins = [((K.float() / dk ** 0.5).to(dtype), V, g, b) for (K, V, g, b) in ins]
    S = [torch.zeros(H, dv, dk, dtype=torch.float32, device="cuda") if S0 is None else S0[l].clone().cuda()
         for l in range(layers)]
    desc = rf.gdn_desc(H, dk, dv, dtype, normalise)
    dev = [[x.cuda() for x in inp] for inp in ins]
    chunks = chunks or [T]
    t0 = 0
    for c in chunks:
        rf.rf_gdn_state(desc, [d[0][t0:t0 + c] for d in dev], [d[1][t0:t0 + c] for d in dev],
                        [d[2][t0:t0 + c] for d in dev], [d[3][t0:t0 + c] for d in dev], S)
        t0 += c
    torch.cuda.synchronize()
    errs = []
    for l, (K, V, g, b) in enumerate(ins):
        ref = oracle.gdn_state(f64(K).reshape(T, H, dk), f64(V).reshape(T, H, dv), f64(g), f64(b),
                               None if S0 is None else f64(S0[l]), normalise_k=normalise)
        assert np.all(np.isfinite(ref)) and bool(torch.isfinite(S[l]).all())
        errs.append(float(np.max(np.abs(f64(S[l]) - ref)) / np.max(np.abs(ref))))
    return errs


@pytest.mark.parametrize("dk,dv,T,dtype,normalise", [
    (128, 128, 300, torch.bfloat16, True),
    (64, 100, 33, torch.float32, True),
    (128, 40, 1, torch.bfloat16, True),
    (64, 64, 97, torch.float32, False),
])
def test_gdn_state_matches_the_recurrence(dk, dv, T, dtype, normalise):
    errs = _run(2, 3, dk, dv, T, dtype, normalise)
    log(f"[gdn] dk={dk} dv={dv} T={T} {dtype} normalise={normalise}: errs={np.round(errs, 7).tolist()}")
    assert max(errs) <= GDN_TOL


def test_gdn_state_chunked_continuation_and_initial_state():
    # a prompt in uneven chunks continues from each chunk's state, starting from a given state
    H, dk, dv, T = 2, 128, 128, 260
    S0 = [torch.randn(H, dv, dk, generator=synth.generator(7, "gdn-S0", l)) * 0.3 for l in range(3)]
    errs = _run(3, H, dk, dv, T, torch.bfloat16, True, chunks=[31, 100, 1, 128], S0=S0)
    log(f"[gdn] chunks 31/100/1/128 from a given state: errs={np.round(errs, 7).tolist()}")
    assert max(errs) <= GDN_TOL


def test_gdn_state_strong_and_mild_decay_blocks():
    # the kernel carries a block's state scaled by its running decay only while that decay stays
    # within 2^-60..2^60, and runs the direct form otherwise: 32-token blocks alternate between
    # mild decays (scaled) and decays of e^-3 per token (direct), a ragged tail ends mild, and
    # one block mixes both near its end (the bound reached inside the block), from a given state
    import linear_kv_cache_amd as rf
    H, dk, dv, T = 2, 128, 64, 32 * 7 + 13
    K, V, g, b = synth.gdn_inputs(13, 0, T, H, dk, dv, torch.bfloat16)
    blk = torch.arange(T) // 32
    g = torch.where((blk % 2 == 1)[:, None], torch.full_like(g, -3.0), g)
    g[32 * 4 + 20:32 * 5] = -4.0        # block 4: mild, then strong from token 20 on
    S0 = torch.randn(H, dv, dk, generator=synth.generator(13, "gdn-S0")) * 0.3
    S = [S0.clone().cuda()]
    rf.rf_gdn_state(rf.gdn_desc(H, dk, dv, torch.bfloat16, True), [K.cuda()], [V.cuda()], [g.cuda()], [b.cuda()], S)
    torch.cuda.synchronize()
    ref = oracle.gdn_state(f64(K).reshape(T, H, dk), f64(V).reshape(T, H, dv), f64(g), f64(b), f64(S0),
                           normalise_k=True)
    err = float(np.max(np.abs(f64(S[0]) - ref)) / np.max(np.abs(ref)))
    log(f"[gdn] strong and mild decay blocks: err={err:.3g}")
    assert bool(torch.isfinite(S[0]).all()) and err <= GDN_TOL


@pytest.mark.slow
@pytest.mark.timeout(300)
def test_gdn_state_full_prompt_sampled_heads():
    # 4 layers x 16 heads x (128 x 128) states over a 16384-token prompt; the oracle checks two
    # heads of the first and last layer (the heads are independent, so a head's inputs alone
    # define its state)
    import linear_kv_cache_amd as rf
    L, H, dk, dv, T = 4, 16, 128, 128, 16384
    ins = [synth.gdn_inputs(11, l, T, H, dk, dv, torch.bfloat16, device="cuda") for l in range(L)]
    S = [torch.zeros(H, dv, dk, dtype=torch.float32, device="cuda") for _ in range(L)]
    rf.rf_gdn_state(rf.gdn_desc(H, dk, dv, torch.bfloat16, True), [x[0] for x in ins], [x[1] for x in ins],
                    [x[2] for x in ins], [x[3] for x in ins], S)
    torch.cuda.synchronize()
    errs = []
    for l in (0, L - 1):
        K, V, g, b = (f64(x) for x in ins[l])
        for h in (0, 9):
            ref = oracle.gdn_state(K.reshape(T, H, dk)[:, h:h + 1], V.reshape(T, H, dv)[:, h:h + 1], g[:, h:h + 1],
                                   b[:, h:h + 1], normalise_k=True)[0]
            errs.append(float(np.max(np.abs(f64(S[l][h]) - ref)) / np.max(np.abs(ref))))
    log(f"[gdn] full prompt T={T}: errs={np.round(errs, 7).tolist()}")
    assert max(errs) <= GDN_TOL
    assert all(bool(torch.isfinite(s).all()) for s in S)
