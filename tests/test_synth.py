"""The seeded generators are deterministic, chunk-addressable and follow their stated laws."""
import torch

import synth


def test_deterministic_and_chunk_addressable():
    cfg = synth.scaled(synth.C2, d=64)
    a = synth.hidden_states(cfg, 32, "calib", chunk=3)
    b = synth.hidden_states(cfg, 32, "calib", chunk=3)
    c = synth.hidden_states(cfg, 32, "calib", chunk=4)
    assert a.dtype == torch.bfloat16 and torch.equal(a, b) and not torch.equal(a, c)


def test_laws():
    cfg = synth.scaled(synth.C5, d=1000)
    s = synth.channel_scales(cfg)
    assert int((s == 20).sum()) == 10 and int((s == 1).sum()) == 990
    cfg2 = synth.scaled(synth.C2, d=256, dtype="f32")
    X = synth.hidden_states(cfg2, 4096, "calib")
    Y = synth.late_layer_inputs(cfg2, X, 16)
    perm, sign = synth.signed_permutation(cfg2, 16)
    resid = Y - X - 0.02 * X[:, perm] * sign
    assert abs(float(resid.std()) - 0.1) < 0.005
    W, b = synth.law_map(cfg2, 16)
    assert W.shape == (256, 256) and abs(float(W.diagonal().mean()) - 1) < 0.01
    bt = synth.block_table(synth.C5, 100)
    assert bt.dtype == torch.int32 and len(set(bt.tolist())) == len(bt) == 7
