"""Python binding of libridgefill (RidgeFill ridge fit and late-layer KV-cache fill, gfx950).

Argument marshalling only: every function forwards to the C entry point of the same name in
``libridgefill.so`` (declared in ``include/ridgefill.h``).  Tensors are passed as device
pointers, streams as ``hipStream_t`` handles; nothing is computed in Python.  PyTorch is used
for device memory and streams only.

The library must have been built (``python linear_kv_cache_amd/build.py``); importing this
module without it raises ImportError.  There is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libridgefill.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"libridgefill.so is not built ({LIB_PATH}); run `python linear_kv_cache_amd/build.py`")
_lib = C.CDLL(LIB_PATH)

# ---- enums (ridgefill.h) -------------------------------------------------------------------
RF_OK, RF_ERR_INVALID_ARG, RF_ERR_UNSUPPORTED, RF_ERR_HIP, RF_ERR_WORKSPACE, RF_ERR_NOT_SPD = range(6)
RF_F32, RF_BF16 = 0, 1
RF_LAYOUT_CONTIGUOUS, RF_LAYOUT_PAGED = 0, 1
RF_LAMBDA_ABSOLUTE, RF_LAMBDA_REL_MEAN_DIAG = 0, 1
RF_PRODUCT_AUTO, RF_PRODUCT_SPLIT_BF16, RF_PRODUCT_F64 = 0, 1, 2
RF_SPLIT_COND_MAX = 8.0
RF_MAX_LAMBDAS = 8

_STATUS = {0: "RF_OK", 1: "RF_ERR_INVALID_ARG", 2: "RF_ERR_UNSUPPORTED", 3: "RF_ERR_HIP", 4: "RF_ERR_WORKSPACE",
           5: "RF_ERR_NOT_SPD"}


class RidgeFillError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status
        self.message = message


# ---- structs -------------------------------------------------------------------------------
class rf_gram_desc(C.Structure):
    _fields_ = [("d", C.c_int32), ("n_targets", C.c_int32), ("dtype", C.c_int), ("d_out", C.c_int32)]


class rf_gram_layout_t(C.Structure):
    _fields_ = [(n, C.c_int64) for n in ("off_n", "off_S_xx", "off_S_yx", "off_s_x", "off_s_y", "off_s_yy",
                                          "total_bytes")]


class rf_cache_desc(C.Structure):
    _fields_ = [("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("block_size", C.c_int32),
                ("max_tokens", C.c_int64), ("layout", C.c_int), ("dtype", C.c_int)]


class rf_cache_layout_t(C.Structure):
    _fields_ = [(n, C.c_int64) for n in ("n_blocks", "elem_bytes", "bytes_per_pool", "stride_block",
                                          "stride_head", "stride_token")]


class rf_fill_weights(C.Structure):
    _fields_ = [("d", C.c_int32), ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("rms_eps", C.c_float),
                ("dtype", C.c_int), ("W_map", C.POINTER(C.c_void_p)), ("b_map", C.POINTER(C.c_void_p)),
                ("gamma", C.POINTER(C.c_void_p)), ("W_k", C.POINTER(C.c_void_p)), ("W_v", C.POINTER(C.c_void_p)),
                ("k_norm", C.POINTER(C.c_void_p)), ("k_norm_eps", C.c_float), ("map_scale", C.POINTER(C.c_void_p)),
                ("rope_base", C.c_double)]


class rf_fill_composed_weights(C.Structure):
    _fields_ = [("d", C.c_int32), ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("rms_eps", C.c_float),
                ("T", C.POINTER(C.c_void_p)), ("q", C.POINTER(C.c_void_p)), ("M_k", C.POINTER(C.c_void_p)),
                ("M_v", C.POINTER(C.c_void_p)), ("c_k", C.POINTER(C.c_void_p)), ("c_v", C.POINTER(C.c_void_p)),
                ("k_norm", C.POINTER(C.c_void_p)), ("k_norm_eps", C.c_float), ("rope_base", C.c_double)]


class rf_gdn_desc(C.Structure):
    _fields_ = [("n_heads", C.c_int32), ("d_k", C.c_int32), ("d_v", C.c_int32), ("dtype", C.c_int),
                ("normalise_k", C.c_int32), ("eps", C.c_float)]


class rf_translate_weights(C.Structure):
    _fields_ = [("d_in", C.c_int32), ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("dtype", C.c_int),
                ("T_k", C.POINTER(C.c_void_p)), ("T_v", C.POINTER(C.c_void_p)), ("b_k", C.POINTER(C.c_void_p)),
                ("b_v", C.POINTER(C.c_void_p)), ("headwise", C.c_int32), ("k_norm", C.POINTER(C.c_void_p)),
                ("k_norm_eps", C.c_float)]


_P = C.c_void_p
_sig = {
    "rf_version": (C.c_char_p, []),
    "rf_last_error": (C.c_char_p, []),
    "rf_gram_state_layout": (C.c_int, [C.POINTER(rf_gram_desc), C.POINTER(rf_gram_layout_t)]),
    "rf_gram_state_bytes": (C.c_size_t, [C.POINTER(rf_gram_desc)]),
    "rf_gram_init": (C.c_int, [C.POINTER(rf_gram_desc), _P, _P]),
    "rf_gram_accumulate": (C.c_int, [C.POINTER(rf_gram_desc), _P, _P, C.c_int64, C.POINTER(_P), C.c_int64,
                                     C.c_int64, _P]),
    "rf_gram_select": (C.c_int, [C.POINTER(rf_gram_desc), _P, C.c_int32, C.POINTER(C.c_int32), C.c_int32,
                                 C.POINTER(rf_gram_desc), _P, _P]),
    "rf_solve_workspace_bytes": (C.c_size_t, [C.POINTER(rf_gram_desc), C.c_int32, C.c_int32]),
    "rf_solve": (C.c_int, [C.POINTER(rf_gram_desc), _P, C.POINTER(C.c_double), C.c_int32, C.c_int,
                           C.POINTER(C.c_int32), C.c_int32, C.c_int, _P, _P, _P, _P, _P, _P, _P, C.c_size_t, _P]),
    "rf_solve_headwise": (C.c_int, [C.POINTER(rf_gram_desc), _P, C.POINTER(C.c_double), C.c_int32, C.c_int,
                                    C.c_int32, C.POINTER(C.c_int32), C.c_int32, C.c_int, _P, _P, _P, _P, _P, _P, _P,
                                    C.c_size_t, _P]),
    "rf_info_status": (C.c_int, [C.POINTER(C.c_int32), C.c_int32]),
    "rf_solve_pinv_workspace_bytes": (C.c_size_t, [C.POINTER(rf_gram_desc), C.c_int32]),
    "rf_solve_pinv": (C.c_int, [C.POINTER(rf_gram_desc), _P, C.c_double, C.c_int, C.c_double, C.c_int32,
                                C.POINTER(C.c_int32), C.c_int32, _P, _P, _P, _P, C.c_size_t, _P]),
    "rf_cache_layout": (C.c_int, [C.POINTER(rf_cache_desc), C.POINTER(rf_cache_layout_t)]),
    "rf_rope_table": (C.c_int, [C.c_double, C.c_int32, C.c_int64, _P, _P]),
    "rf_pack_weights": (C.c_int, [C.c_int, C.c_int64, C.c_int64, _P, C.c_int64, C.c_int32, _P, _P]),
    "rf_quantize_map": (C.c_int, [C.c_int64, C.c_int64, _P, C.c_int64, _P, _P, _P]),
    "rf_rope_workspace_bytes": (C.c_size_t, [C.c_int32, C.c_int64]),
    "rf_fill_workspace_bytes": (C.c_size_t, [C.POINTER(rf_fill_weights), C.c_int64]),
    "rf_fill": (C.c_int, [C.POINTER(rf_fill_weights), C.c_int32, _P, C.c_int64, C.c_int64, C.c_int64, C.c_int64,
                          C.POINTER(rf_cache_desc), C.POINTER(_P), C.POINTER(_P), _P, C.c_int64, _P, C.c_int64,
                          _P, C.c_size_t, _P]),
    "rf_translate": (C.c_int, [C.POINTER(rf_translate_weights), C.c_int32, C.POINTER(_P), C.POINTER(_P), C.c_int64,
                               C.c_int64, C.c_int64, C.c_int64, C.POINTER(rf_cache_desc), C.POINTER(_P),
                               C.POINTER(_P), _P, C.c_int64, _P, C.c_int64, _P]),
    "rf_relative_depth_sources": (C.c_int, [C.c_int32, C.c_int32, C.c_int32, C.POINTER(C.c_int32)]),
    "rf_fill_compose_workspace_bytes": (C.c_size_t, [C.POINTER(rf_fill_weights)]),
    "rf_fill_compose": (C.c_int, [C.POINTER(rf_fill_weights), C.c_int32, C.POINTER(_P), C.POINTER(_P), C.POINTER(_P),
                                  C.POINTER(_P), C.POINTER(_P), C.POINTER(_P), _P, C.c_size_t, _P]),
    "rf_fill_composed_workspace_bytes": (C.c_size_t, [C.POINTER(rf_fill_composed_weights), C.c_int64]),
    "rf_fill_composed": (C.c_int, [C.POINTER(rf_fill_composed_weights), C.c_int32, _P, C.c_int64, C.c_int64,
                                   C.c_int64, C.c_int64, C.POINTER(rf_cache_desc), C.POINTER(_P), C.POINTER(_P), _P,
                                   C.c_int64, _P, C.c_int64, _P, C.c_size_t, _P]),
    "rf_gdn_state": (C.c_int, [C.POINTER(rf_gdn_desc), C.c_int32, C.POINTER(_P), C.POINTER(_P), C.c_int64, C.c_int64,
                               C.POINTER(_P), C.POINTER(_P), C.c_int64, C.POINTER(_P), _P]),
    "rf_fill_static_scratch_bytes": (C.c_size_t, []),
    "rf_fill_static": (C.c_int, [C.POINTER(rf_fill_weights), C.c_int32, _P, C.c_int64, C.c_int64, C.c_int64,
                                 C.c_int64, C.POINTER(rf_cache_desc), C.POINTER(_P), C.POINTER(_P), _P, C.c_int64, _P,
                                 C.c_int64, _P]),
    "rf_fill_streamed_ring_bytes": (C.c_size_t, [C.POINTER(rf_fill_weights), C.c_int32, C.c_int32]),
    "rf_fill_streamed": (C.c_int, [C.POINTER(rf_fill_weights), C.c_int32, _P, C.c_int64, C.c_int64, C.c_int64,
                                   C.c_int64, C.POINTER(rf_cache_desc), C.POINTER(_P), C.POINTER(_P), _P, C.c_int64, _P,
                                   C.c_int64, _P, C.c_size_t, _P, C.c_size_t, C.c_int32, C.c_int32, C.c_int64, _P, _P]),
    "rf_fit_r2_workspace_bytes": (C.c_size_t, [C.POINTER(rf_gram_desc), C.c_int32]),
    "rf_fit_r2": (C.c_int, [C.POINTER(rf_gram_desc), _P, C.c_double, C.c_int, C.POINTER(C.c_int32), C.c_int32, _P, _P,
                            _P, C.c_size_t, _P]),
    "rf_r2_assignment": (C.c_int, [C.POINTER(C.c_double), C.c_int32, C.c_int32, C.c_int32, C.POINTER(C.c_int32)]),
}
for _name, (_res, _args) in _sig.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args

EXPORTED = tuple(_sig)


def _check(status: int):
    if status != RF_OK:
        raise RidgeFillError(status, _lib.rf_last_error().decode())


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(s) -> Optional[int]:
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _ptr_array(xs) -> C.Array:
    arr = (_P * max(1, len(xs)))()
    for i, x in enumerate(xs):
        arr[i] = _ptr(x)
    return arr


def _dtype_code(t) -> int:
    import torch
    if t == torch.float32 or t == RF_F32:
        return RF_F32
    if t == torch.bfloat16 or t == RF_BF16:
        return RF_BF16
    raise ValueError(f"unsupported dtype {t}")


# ---- API ------------------------------------------------------------------------------------
def rf_version() -> str:
    return _lib.rf_version().decode()


def rf_last_error() -> str:
    return _lib.rf_last_error().decode()


def gram_desc(d: int, n_targets: int, dtype, d_out: int = 0) -> rf_gram_desc:
    """d_out: width of each target's rows (0 = d)."""
    return rf_gram_desc(d, n_targets, _dtype_code(dtype), d_out)


def rf_gram_state_layout(desc: rf_gram_desc) -> dict:
    out = rf_gram_layout_t()
    _check(_lib.rf_gram_state_layout(C.byref(desc), C.byref(out)))
    return {n: getattr(out, n) for n, _ in rf_gram_layout_t._fields_}


def rf_gram_state_bytes(desc: rf_gram_desc) -> int:
    return int(_lib.rf_gram_state_bytes(C.byref(desc)))


def rf_gram_init(desc: rf_gram_desc, state, stream=None):
    _check(_lib.rf_gram_init(C.byref(desc), _ptr(state), _stream(stream)))


def rf_gram_accumulate(desc: rf_gram_desc, state, X, Ys: Sequence, rows: Optional[int] = None, stream=None):
    """X: [rows, >=d] tensor (row stride = ldx); Ys: n_targets tensors [rows, >=d_out] sharing one row stride."""
    rows = X.shape[0] if rows is None else rows
    ldy = Ys[0].stride(0) if len(Ys) else desc.d
    if any(Y.stride(0) != ldy for Y in Ys):
        raise ValueError("all Y tensors must share one row stride")
    ys = _ptr_array(Ys)
    _check(_lib.rf_gram_accumulate(C.byref(desc), _ptr(state), _ptr(X), X.stride(0), ys, ldy, rows,
                                   _stream(stream)))


def rf_gram_select(desc: rf_gram_desc, state, block_width: int, blocks: Sequence[int], desc_out: rf_gram_desc,
                   state_out, stream=None):
    bl = (C.c_int32 * max(1, len(blocks)))(*blocks)
    _check(_lib.rf_gram_select(C.byref(desc), _ptr(state), block_width, bl, len(blocks), C.byref(desc_out),
                               _ptr(state_out), _stream(stream)))


def rf_solve_workspace_bytes(desc: rf_gram_desc, n_sel: int, n_lambda: int = 1) -> int:
    return int(_lib.rf_solve_workspace_bytes(C.byref(desc), n_sel, n_lambda))


def rf_solve(desc: rf_gram_desc, state, lambdas, mode: int, targets: Sequence[int], W, W_lp, b, info, ws,
             stream=None, product: int = RF_PRODUCT_AUTO, cond=None, resid=None):
    """lambdas: one ridge strength or a sequence of up to 8 (the outputs gain a leading axis)."""
    lams = [float(lambdas)] if isinstance(lambdas, (int, float)) else [float(x) for x in lambdas]
    la = (C.c_double * max(1, len(lams)))(*lams)
    tg = (C.c_int32 * max(1, len(targets)))(*targets)
    ws_bytes = ws.numel() * ws.element_size()
    _check(_lib.rf_solve(C.byref(desc), _ptr(state), la, len(lams), int(mode), tg, len(targets), int(product), _ptr(W),
                         _ptr(W_lp), _ptr(b), _ptr(info), _ptr(cond), _ptr(resid), _ptr(ws), ws_bytes,
                         _stream(stream)))


def rf_solve_headwise(desc: rf_gram_desc, state, lambdas, mode: int, head_dim: int, targets: Sequence[int], W, W_lp,
                      b, info, ws, stream=None, product: int = RF_PRODUCT_AUTO, cond=None, resid=None):
    """rf_solve for maps block-diagonal by head (one ridge fit per head); arguments as rf_solve."""
    lams = [float(lambdas)] if isinstance(lambdas, (int, float)) else [float(x) for x in lambdas]
    la = (C.c_double * max(1, len(lams)))(*lams)
    tg = (C.c_int32 * max(1, len(targets)))(*targets)
    ws_bytes = ws.numel() * ws.element_size()
    _check(_lib.rf_solve_headwise(C.byref(desc), _ptr(state), la, len(lams), int(mode), int(head_dim), tg,
                                  len(targets), int(product), _ptr(W), _ptr(W_lp), _ptr(b), _ptr(info), _ptr(cond),
                                  _ptr(resid), _ptr(ws), ws_bytes, _stream(stream)))


def rf_info_status(info: Sequence[int]) -> int:
    """RF_OK, or RF_ERR_NOT_SPD (message in rf_last_error()) for a host copy of rf_solve's pivots."""
    arr = (C.c_int32 * max(1, len(info)))(*[int(x) for x in info])
    return int(_lib.rf_info_status(arr, len(info)))


def rf_solve_pinv_workspace_bytes(desc: rf_gram_desc, n_sel: int) -> int:
    return int(_lib.rf_solve_pinv_workspace_bytes(C.byref(desc), n_sel))


def rf_solve_pinv(desc: rf_gram_desc, state, lam: float, mode: int, rel_tol: float, sweeps: int,
                  targets: Sequence[int], W, W_lp, b, ws, stream=None):
    tg = (C.c_int32 * max(1, len(targets)))(*targets)
    ws_bytes = ws.numel() * ws.element_size()
    _check(_lib.rf_solve_pinv(C.byref(desc), _ptr(state), float(lam), int(mode), float(rel_tol), int(sweeps), tg,
                              len(targets), _ptr(W), _ptr(W_lp), _ptr(b), _ptr(ws), ws_bytes, _stream(stream)))


def cache_desc(n_kv_heads: int, head_dim: int, max_tokens: int, layout: int, dtype, block_size: int = 16):
    return rf_cache_desc(n_kv_heads, head_dim, block_size, max_tokens, layout, _dtype_code(dtype))


def rf_cache_layout(desc: rf_cache_desc) -> dict:
    out = rf_cache_layout_t()
    _check(_lib.rf_cache_layout(C.byref(desc), C.byref(out)))
    return {n: getattr(out, n) for n, _ in rf_cache_layout_t._fields_}


def rf_rope_table(base: float, head_dim: int, n_pos: int, table, stream=None):
    _check(_lib.rf_rope_table(float(base), head_dim, n_pos, _ptr(table), _stream(stream)))


def rf_pack_weights(W, dst, rope_head_dim: int = 0, stream=None):
    """W: [rows, >=cols] bf16 or fp32 tensor (row stride = ld_src); dst: rows*cols bf16 elements."""
    rows, cols = W.shape
    _check(_lib.rf_pack_weights(_dtype_code(W.dtype), rows, cols, _ptr(W), W.stride(0), int(rope_head_dim), _ptr(dst),
                                _stream(stream)))


def rf_rope_workspace_bytes(head_dim: int, n_tokens: int) -> int:
    return int(_lib.rf_rope_workspace_bytes(head_dim, n_tokens))


def rf_quantize_map(W, q, scale, stream=None):
    """W: [rows, >=cols] fp32 map (row stride = ld); q: rows*cols int8 codes out (packed);
    scale: [rows] fp32 out."""
    rows, cols = W.shape
    _check(_lib.rf_quantize_map(rows, cols, _ptr(W), W.stride(0), _ptr(q), _ptr(scale), _stream(stream)))


@dataclass
class FillWeights:
    """Per-layer weights of the layers one rf_fill call fills (tensors on the device).

    BF16 weights are in the packed layout: maps as rf_pack_weights(rope_head_dim=0) or
    rf_solve's bf16 output leave them, W_k and W_v as rf_pack_weights(rope_head_dim=head_dim).
    With ``map_scale`` (a list of [d] fp32 tensors) the maps are int8 codes of rf_quantize_map."""

    d: int
    n_kv_heads: int
    head_dim: int
    rms_eps: float
    dtype: object
    W_map: list
    b_map: list
    gamma: list
    W_k: list
    W_v: list
    k_norm: Optional[list] = None
    k_norm_eps: float = 1e-6
    map_scale: Optional[list] = None
    rope_base: float = 0.0   # used only by fills given no RoPE table

    def _c(self):
        arrs = [_ptr_array(x) for x in (self.W_map, self.b_map, self.gamma, self.W_k, self.W_v)]
        kn = None if self.k_norm is None else _ptr_array(self.k_norm)
        ms = None if self.map_scale is None else _ptr_array(self.map_scale)
        w = rf_fill_weights(self.d, self.n_kv_heads, self.head_dim, self.rms_eps, _dtype_code(self.dtype),
                            *[C.cast(a, C.POINTER(_P)) for a in arrs],
                            C.cast(kn, C.POINTER(_P)) if kn is not None else C.POINTER(_P)(), self.k_norm_eps,
                            C.cast(ms, C.POINTER(_P)) if ms is not None else C.POINTER(_P)(), float(self.rope_base))
        return w, (arrs, kn, ms)


def rf_fill_workspace_bytes(weights: FillWeights, max_rows: int) -> int:
    w, _keep = weights._c()
    return int(_lib.rf_fill_workspace_bytes(C.byref(w), max_rows))


def rf_fill(weights: FillWeights, X, t0: int, t1: int, pos0: int, cache: rf_cache_desc, k_cache: Sequence,
            v_cache: Sequence, block_table, rope, rope_len: int, ws, stream=None, n_layers: Optional[int] = None):
    w, _keep = weights._c()
    n_layers = len(weights.W_map) if n_layers is None else n_layers
    kc = _ptr_array(k_cache)
    vc = _ptr_array(v_cache)
    n_tab = 0 if block_table is None else block_table.numel()
    ws_bytes = ws.numel() * ws.element_size()
    _check(_lib.rf_fill(C.byref(w), n_layers, _ptr(X), X.stride(0), t0, t1, pos0, C.byref(cache), kc, vc,
                        _ptr(block_table), n_tab, _ptr(rope), rope_len, _ptr(ws), ws_bytes, _stream(stream)))


@dataclass
class ComposedFillWeights:
    """Per-layer composed weights of one rf_fill_composed call (tensors on the device), as
    rf_fill_compose writes them: T [d, d] and M_k, M_v [H*d_h, d] packed bf16; q [2d + 1], c_k,
    c_v [H*d_h] fp32."""

    d: int
    n_kv_heads: int
    head_dim: int
    rms_eps: float
    T: list
    q: list
    M_k: list
    M_v: list
    c_k: list
    c_v: list
    k_norm: Optional[list] = None
    k_norm_eps: float = 1e-6
    rope_base: float = 0.0   # used only by fills given no RoPE table

    def _c(self):
        arrs = [_ptr_array(x) for x in (self.T, self.q, self.M_k, self.M_v, self.c_k, self.c_v)]
        kn = None if self.k_norm is None else _ptr_array(self.k_norm)
        w = rf_fill_composed_weights(self.d, self.n_kv_heads, self.head_dim, self.rms_eps,
                                     *[C.cast(a, C.POINTER(_P)) for a in arrs],
                                     C.cast(kn, C.POINTER(_P)) if kn is not None else C.POINTER(_P)(), self.k_norm_eps,
                                     float(self.rope_base))
        return w, (arrs, kn)


def rf_fill_compose_workspace_bytes(weights: FillWeights) -> int:
    w, _keep = weights._c()
    return int(_lib.rf_fill_compose_workspace_bytes(C.byref(w)))


def rf_fill_compose(weights: FillWeights, out: ComposedFillWeights, ws, stream=None, n_layers: Optional[int] = None):
    """Composed weights of the listed layers into the buffers of ``out``."""
    w, _keep = weights._c()
    n_layers = len(weights.W_map) if n_layers is None else n_layers
    arrs = [_ptr_array(x) for x in (out.T, out.q, out.M_k, out.M_v, out.c_k, out.c_v)]
    ws_bytes = ws.numel() * ws.element_size()
    _check(_lib.rf_fill_compose(C.byref(w), n_layers, *arrs, _ptr(ws), ws_bytes, _stream(stream)))


def rf_fill_composed_workspace_bytes(weights: ComposedFillWeights, max_rows: int) -> int:
    w, _keep = weights._c()
    return int(_lib.rf_fill_composed_workspace_bytes(C.byref(w), max_rows))


def rf_fill_composed(weights: ComposedFillWeights, X, t0: int, t1: int, pos0: int, cache: rf_cache_desc,
                     k_cache: Sequence, v_cache: Sequence, block_table, rope, rope_len: int, ws, stream=None,
                     n_layers: Optional[int] = None):
    w, _keep = weights._c()
    n_layers = len(weights.T) if n_layers is None else n_layers
    kc = _ptr_array(k_cache)
    vc = _ptr_array(v_cache)
    n_tab = 0 if block_table is None else block_table.numel()
    ws_bytes = ws.numel() * ws.element_size()
    _check(_lib.rf_fill_composed(C.byref(w), n_layers, _ptr(X), X.stride(0), t0, t1, pos0, C.byref(cache), kc, vc,
                                 _ptr(block_table), n_tab, _ptr(rope), rope_len, _ptr(ws), ws_bytes, _stream(stream)))


def gdn_desc(n_heads: int, d_k: int, d_v: int, dtype, normalise_k: bool = True, eps: float = 1e-6) -> rf_gdn_desc:
    return rf_gdn_desc(n_heads, d_k, d_v, _dtype_code(dtype), int(bool(normalise_k)), eps)


def rf_gdn_state(desc: rf_gdn_desc, K: Sequence, V: Sequence, g: Sequence, beta: Sequence, states: Sequence,
                 n_tokens: Optional[int] = None, stream=None):
    """K, V: per layer [n_tokens, >= n_heads*d_k] / [n_tokens, >= n_heads*d_v] tensors (one row
    stride for all K, one for all V); g, beta: per layer [n_tokens, n_heads] fp32; states: per
    layer [n_heads, d_v, d_k] fp32, updated in place."""
    n = K[0].shape[0] if n_tokens is None else n_tokens
    _check(_lib.rf_gdn_state(C.byref(desc), len(K), _ptr_array(K), _ptr_array(V), K[0].stride(0), V[0].stride(0),
                             _ptr_array(g), _ptr_array(beta), n, _ptr_array(states), _stream(stream)))


def rf_fill_static_scratch_bytes() -> int:
    return int(_lib.rf_fill_static_scratch_bytes())


def rf_fill_static(weights: FillWeights, X, t0: int, t1: int, pos0: int, cache: rf_cache_desc, k_cache: Sequence,
                   v_cache: Sequence, block_table, rope, rope_len: int, stream=None, n_layers: Optional[int] = None):
    """rf_fill with the library's static scratch buffer instead of a workspace argument."""
    w, _keep = weights._c()
    n_layers = len(weights.W_map) if n_layers is None else n_layers
    kc = _ptr_array(k_cache)
    vc = _ptr_array(v_cache)
    n_tab = 0 if block_table is None else block_table.numel()
    _check(_lib.rf_fill_static(C.byref(w), n_layers, _ptr(X), X.stride(0), t0, t1, pos0, C.byref(cache), kc, vc,
                               _ptr(block_table), n_tab, _ptr(rope), rope_len, _stream(stream)))


@dataclass
class TranslateWeights:
    """Per-target-layer translator maps of one rf_translate call (tensors on the device).

    T_k, T_v: [n_kv_heads*head_dim, d_in] out-feature major; BF16 maps packed by
    rf_pack_weights(rope_head_dim=head_dim).  b_k, b_v: lists of fp32 intercepts, or None.
    headwise: the maps are block-diagonal by head (only the head blocks are read)."""

    d_in: int
    n_kv_heads: int
    head_dim: int
    dtype: object
    T_k: list
    T_v: list
    b_k: Optional[list] = None
    b_v: Optional[list] = None
    headwise: bool = False
    k_norm: Optional[list] = None
    k_norm_eps: float = 1e-6

    def _c(self):
        arrs = [_ptr_array(x) for x in (self.T_k, self.T_v)]
        barrs = [None if x is None else _ptr_array(x) for x in (self.b_k, self.b_v, self.k_norm)]
        cast = lambda a: C.cast(a, C.POINTER(_P)) if a is not None else C.POINTER(_P)()
        w = rf_translate_weights(self.d_in, self.n_kv_heads, self.head_dim, _dtype_code(self.dtype),
                                 cast(arrs[0]), cast(arrs[1]), cast(barrs[0]), cast(barrs[1]), int(self.headwise),
                                 cast(barrs[2]), self.k_norm_eps)
        return w, (arrs, barrs)


def rf_translate(weights: TranslateWeights, src_k: Sequence, src_v: Sequence, ld_src: int, t0: int, t1: int,
                 pos0: int, cache: rf_cache_desc, k_cache: Sequence, v_cache: Sequence, block_table, rope,
                 rope_len: int, stream=None, n_layers: Optional[int] = None):
    """src_k, src_v: per target layer, device pointers (or tensors) to the source rows of token t0."""
    w, _keep = weights._c()
    n_layers = len(weights.T_k) if n_layers is None else n_layers
    n_tab = 0 if block_table is None else block_table.numel()
    _check(_lib.rf_translate(C.byref(w), n_layers, _ptr_array(src_k), _ptr_array(src_v), ld_src, t0, t1, pos0,
                             C.byref(cache), _ptr_array(k_cache), _ptr_array(v_cache), _ptr(block_table), n_tab,
                             _ptr(rope), rope_len, _stream(stream)))


def rf_fill_streamed_ring_bytes(weights: FillWeights, ring_slots: int, layers_per_slot: int) -> int:
    w, _keep = weights._c()
    return int(_lib.rf_fill_streamed_ring_bytes(C.byref(w), ring_slots, layers_per_slot))


def rf_fill_streamed(weights: FillWeights, X, t0: int, t1: int, pos0: int, cache: rf_cache_desc, k_cache: Sequence,
                     v_cache: Sequence, block_table, rope, rope_len: int, ws, ring, ring_slots: int,
                     layers_per_slot: int, stream, copy_stream, n_layers: Optional[int] = None, rows_per_fill: int = 0):
    """weights.W_map: pinned host tensors (the maps); everything else on the device.
    rows_per_fill: tokens per fill step inside each layer chunk (0 = the whole range)."""
    w, _keep = weights._c()
    n_layers = len(weights.W_map) if n_layers is None else n_layers
    n_tab = 0 if block_table is None else block_table.numel()
    _check(_lib.rf_fill_streamed(C.byref(w), n_layers, _ptr(X), X.stride(0), t0, t1, pos0, C.byref(cache),
                                 _ptr_array(k_cache), _ptr_array(v_cache), _ptr(block_table), n_tab, _ptr(rope),
                                 rope_len, _ptr(ws), ws.numel() * ws.element_size(), _ptr(ring),
                                 ring.numel() * ring.element_size(), ring_slots, layers_per_slot, rows_per_fill,
                                 _stream(stream), _stream(copy_stream)))


def rf_fit_r2_workspace_bytes(desc: rf_gram_desc, n_sel: int) -> int:
    return int(_lib.rf_fit_r2_workspace_bytes(C.byref(desc), n_sel))


def rf_fit_r2(desc: rf_gram_desc, state, lam: float, mode: int, targets: Sequence[int], W, r2, ws, stream=None):
    """W: the fp32 maps rf_solve returned for ``targets``; r2: [n_sel] fp64 device output."""
    tg = (C.c_int32 * max(1, len(targets)))(*targets)
    ws_bytes = ws.numel() * ws.element_size()
    _check(_lib.rf_fit_r2(C.byref(desc), _ptr(state), float(lam), int(mode), tg, len(targets), _ptr(W), _ptr(r2),
                          _ptr(ws), ws_bytes, _stream(stream)))


def rf_r2_assignment(r2_rows: Sequence[Sequence[float]], nu: int) -> list:
    """r2_rows[l][s]: score of source s for target l (host values).  Returns the nu chosen
    source layers of each target, ascending (host only)."""
    n_tgt = len(r2_rows)
    n_src = len(r2_rows[0]) if n_tgt else 0
    flat = (C.c_double * max(1, n_tgt * n_src))(*[float(v) for row in r2_rows for v in row])
    out = (C.c_int32 * max(1, n_tgt * nu))()
    _check(_lib.rf_r2_assignment(flat, n_tgt, n_src, nu, out))
    return [[out[l * nu + j] for j in range(nu)] for l in range(n_tgt)]


def rf_relative_depth_sources(n_src: int, n_tgt: int, nu: int) -> list:
    """0-based source layers of each 0-based target layer (host only)."""
    out = (C.c_int32 * max(1, n_tgt * nu))()
    _check(_lib.rf_relative_depth_sources(n_src, n_tgt, nu, out))
    return [[out[l * nu + j] for j in range(nu)] for l in range(n_tgt)]


__all__ = [n for n in dir() if n.startswith("rf_") or n.startswith("RF_")] + [
    "RidgeFillError", "FillWeights", "TranslateWeights", "gram_desc", "cache_desc", "EXPORTED", "LIB_PATH"]
