"""Pins of the oracle's int8 map quantiser (oracle/quant.py): codes and scales on exact grids,
rounding of ties to even, zero rows, the half-step error bound of the dequantised map, and
invariance under power-of-two scaling.  None of these retypes the quantiser's formula: the
expected codes are written out by hand or follow from the bound."""
import numpy as np

import oracle

S0 = np.float32(2.0 ** -7)   # 127 * 2^-7 / 127 is exactly 2^-7 in fp32


def test_codes_on_an_exact_grid():
    W = S0 * np.array([[127, -64, 3, 0, -127, 1], [-127, 1, 2, 3, 4, 5]], dtype=np.float32)
    q, s = oracle.quantize_rows(W)
    assert q.dtype == np.int8 and s.dtype == np.float32
    assert s.tolist() == [S0, S0]
    assert q.tolist() == [[127, -64, 3, 0, -127, 1], [-127, 1, 2, 3, 4, 5]]
    assert np.array_equal(oracle.dequantize_rows(q, s), W.astype(np.float64))


def test_ties_round_to_even():
    W = S0 * np.array([[127, 2.5, 3.5, -2.5, -0.5, 0.5, 1.5, -126.5]], dtype=np.float32)
    q, s = oracle.quantize_rows(W)
    assert s[0] == S0
    assert q[0].tolist() == [127, 2, 4, -2, 0, 0, 2, -126]


def test_zero_rows_and_a_single_negative_maximum():
    W = np.zeros((3, 5), dtype=np.float32)
    W[1, 3] = -0.75
    q, s = oracle.quantize_rows(W)
    assert s[0] == 0 and s[2] == 0 and not q[0].any() and not q[2].any()
    assert q[1].tolist() == [0, 0, 0, -127, 0]
    assert s[1] == np.float32(0.75) / np.float32(127)


def test_half_step_error_bound_and_full_range():
    rng = np.random.default_rng(11)
    W = (rng.standard_normal((64, 300)) * rng.lognormal(0, 1, (64, 1))).astype(np.float32)
    q, s = oracle.quantize_rows(W)
    err = np.abs(oracle.dequantize_rows(q, s) - W.astype(np.float64))
    # round to nearest: at most half a step, plus the fp32 rounding of W / s (a few ulp)
    assert np.all(err <= s.astype(np.float64)[:, None] * (0.5 + 1e-5))
    assert np.all(np.max(np.abs(q.astype(np.int32)), axis=1) == 127)
    assert np.all(np.abs(q.astype(np.int32)) <= 127)


def test_power_of_two_scaling():
    rng = np.random.default_rng(12)
    W = rng.standard_normal((16, 64)).astype(np.float32)
    q, s = oracle.quantize_rows(W)
    for k in (-20, -3, 5):
        q2, s2 = oracle.quantize_rows(W * np.float32(2.0 ** k))
        assert np.array_equal(q2, q)
        assert np.array_equal(s2, s * np.float32(2.0 ** k))
