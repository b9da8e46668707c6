"""Weight-only int8 maps: the oracle's quantiser.

TEST INFRASTRUCTURE ONLY (see the package docstring).

RidgeFill project page, "Code, data and maps", the table of ridge maps on Hugging Face:
some of the published maps are int8 ("-i8" repositories).  The page writes out no scheme.
The reading taken here: symmetric int8 per output row, weight-only.  Row o of a map W
([d_out][d_in], the layout the fill takes) is stored as a scale s_o and codes q_o with
    s_o = max_i |W[o][i]| / 127,    q[o][i] = round_half_even(W[o][i] / s_o)  in [-127, 127],
and a row of zeros as s_o = 0, q_o = 0; the map the fill applies is then s_o q_o (the
prompt states stay bf16).  A code is an integer that floating point decides, so it is
decided here in the precision of the library's quantiser, fp32 (IEEE division, rounding to
nearest even), not in fp64; the dequantised map is exact in fp64.
"""
import numpy as np


def quantize_rows(W):
    """(q int8 [d_out][d_in], s fp32 [d_out]) of the row-wise symmetric int8 code of W."""
    W32 = np.asarray(W, dtype=np.float32)
    q = np.zeros(W32.shape, dtype=np.int8)
    s = np.zeros(W32.shape[0], dtype=np.float32)
    for o in range(W32.shape[0]):
        amax = np.float32(np.max(np.abs(W32[o]))) if W32.shape[1] else np.float32(0)
        s[o] = amax / np.float32(127.0)
        if s[o] > 0:
            q[o] = np.clip(np.rint(W32[o] / s[o]), -127, 127).astype(np.int8)
    return q, s


def dequantize_rows(q, s) -> np.ndarray:
    """The map the fill applies, s_o q[o][i], in fp64 (exact)."""
    return np.asarray(s, dtype=np.float64)[:, None] * np.asarray(q, dtype=np.float64)
