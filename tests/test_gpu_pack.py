"""The packed weight layout: rf_pack_weights against the layout the header defines, written
out here in NumPy index arithmetic, and the solve's bf16 map against its fp32 map."""
import numpy as np
import pytest
import torch

import synth
from gpu_cases import FitCase, log, run_fit_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def packed_offsets(rows: int, cols: int, hd: int) -> np.ndarray:
    """off[r, k] = element offset of source element (r, k) in the packed buffer."""
    p = np.arange(256)                     # packed row in a tile
    if hd == 0:
        src = p
    else:
        h = hd // 2
        q = 32 * (p // 64) + p % 32
        src = (q // h) * hd + q % h + ((p // 32) % 2) * h
    assert sorted(src.tolist()) == list(range(256))      # a permutation of the tile's rows
    pos = np.empty(256, dtype=np.int64)
    pos[src] = p                           # packed position of each source row
    r = np.arange(rows)[:, None]
    k = np.arange(cols)[None, :]
    rp = pos[r % 256]
    return ((r // 256) * 256 * cols + (k // 64) * 16384 + (rp // 64) * 4096 + ((k % 64) // 16) * 1024
            + ((rp % 64) // 32) * 512 + (((k % 16) // 8) * 32 + rp % 32) * 8 + k % 8)


def unpack(packed: torch.Tensor, rows: int, cols: int, hd: int = 0) -> np.ndarray:
    flat = packed.reshape(-1).view(torch.int16).cpu().numpy()
    return flat[packed_offsets(rows, cols, hd)]


def test_offsets_are_a_bijection():
    for rows, cols, hd in [(256, 64, 0), (512, 192, 64), (256, 128, 128)]:
        off = packed_offsets(rows, cols, hd).ravel()
        assert np.array_equal(np.sort(off), np.arange(rows * cols))


@pytest.mark.parametrize("hd", [0, 64, 128])
def test_pack_matches_layout(hd):
    from linear_kv_cache_amd.runner import pack_weights
    rows, cols, ld = 512, 320, 384
    g = torch.Generator().manual_seed(11 + hd)
    bits = torch.randint(-32768, 32767, (rows, ld), generator=g, dtype=torch.int16)
    W = bits.view(torch.bfloat16).cuda()[:, :cols]
    P = pack_weights(W, hd)
    torch.cuda.synchronize()
    got = unpack(P, rows, cols, hd)
    want = bits[:, :cols].numpy()
    log(f"[pack] hd={hd} rows={rows} cols={cols} ld={ld} mismatches={int(np.sum(got != want))}")
    assert np.array_equal(got, want)


def test_solve_bf16_map_is_the_packed_rounded_map():
    cfg = synth.scaled(synth.C2, name="fit-bf16-d512", d=512, n_layers=6, split=3)
    case = FitCase(cfg, 3000, [3000], 1e-1)
    res = run_fit_case(case)
    assert res["info"] == 0
    W, Wlp = res["W"], res["Wlp"]
    d = cfg.d
    for t in range(W.shape[0]):
        want = W[t].to(torch.bfloat16).view(torch.int16).cpu().numpy()
        got = unpack(Wlp[t], d, d)
        log(f"[pack] solve target {t}: mismatches={int(np.sum(got != want))}")
        assert np.array_equal(got, want)
