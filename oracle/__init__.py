"""Plain fp64 CPU oracle for RidgeFill's ridge fit and late-layer cache fill.

TEST INFRASTRUCTURE ONLY.  This package is the reference the HIP library is checked
against.  Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
it; the product path (``linear_kv_cache_amd``) never does, and the two share no code.

Everything is computed in float64 with NumPy/SciPy from the stored input values, upcast
exactly.  Sources are the RidgeFill project page ("Method": steps 1-4 and Figure 2;
"Abstract") and, for the pre-norm storing order and the relative ridge convention, the
KV-Lingo page (sections 2 and 3.1, Appendix B.2 "Protocol").  ``translate`` follows the
KV-Lingo page's token-wise linear cache translators (sections 3.1 and 3.2).  ``quantize_rows``
is the reading of the project page's int8 maps ("Code, data and maps") as row-wise
symmetric weight-only codes.

Readings taken where the pages are silent (each one is listed in the design notes):
  * the map is W = (X~^T X~ + lambda I)^-1 X~^T Y~ on mean-centred rows with the intercept
    b = mean(Y) - mean(X) W (the project page says only "ridge regression, fitted once in
    closed form");
  * lambda is absolute, or relative to the mean diagonal of the centred Gram;
  * the late layer's own K/V path is RMSNorm (epsilon inside the root), then the K and V
    projections, then rotate-half RoPE on K with 0-based absolute positions.

Parity status: every function here is pinned by tests/test_oracle_*.py against closed
forms, limits, brute force or an independent library route.  ``gdn_state`` (the Gated
DeltaNet state update, a published recurrence the pages name but do not write out) is pinned
by the recurrence's own closed forms; against the pages its parity is unpinned.
"""
from .ridge import (NotSPD, gram_sums, fit, fit_from_sums, fit_pinv, ridge_objective,
                    solve_columns_from_data, stationarity_residual, stationarity_residual_from_sums)
from .fill import rope_inverse_frequencies, rope_rotate, rmsnorm, fill_layer, fill
from .gdn import gdn_state, l2_normalise
from .quant import quantize_rows, dequantize_rows
from .translate import (relative_depth_centre, relative_depth_sources, headwise_dense,
                        translate_layer, translate, fit_translator, fit_r2, r2_assignment,
                        greedy_sources)

__all__ = ["NotSPD", "gram_sums", "fit", "fit_from_sums", "fit_pinv", "ridge_objective",
           "solve_columns_from_data", "stationarity_residual", "stationarity_residual_from_sums",
           "rope_inverse_frequencies", "rope_rotate", "rmsnorm",
           "fill_layer", "fill", "relative_depth_centre", "relative_depth_sources",
           "headwise_dense", "translate_layer", "translate", "fit_translator", "fit_r2",
           "r2_assignment", "greedy_sources", "gdn_state", "l2_normalise", "quantize_rows",
           "dequantize_rows"]
