"""Device-memory plumbing around the C entry points: allocate states, workspaces, caches and
RoPE tables with torch, then call the library.  No arithmetic of the method happens here."""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import List, Optional, Sequence

import torch

from . import (RF_LAYOUT_CONTIGUOUS, RF_LAYOUT_PAGED, RF_PRODUCT_AUTO, ComposedFillWeights, FillWeights, TranslateWeights, cache_desc, gram_desc,
               rf_cache_layout, rf_fill, rf_fill_compose, rf_fill_compose_workspace_bytes, rf_fill_composed,
               rf_fill_composed_workspace_bytes, rf_fill_streamed, rf_fill_streamed_ring_bytes, rf_fill_workspace_bytes,
               rf_fit_r2, rf_fit_r2_workspace_bytes, rf_gram_select,
               rf_gram_accumulate, rf_gram_init,
               rf_gram_state_bytes, rf_gram_state_layout, rf_pack_weights, rf_quantize_map, rf_rope_table, rf_solve,
               rf_solve_headwise, rf_solve_pinv, rf_solve_pinv_workspace_bytes, rf_solve_workspace_bytes,
               rf_translate)


def device_bytes(n: int, device) -> torch.Tensor:
    """A 256-byte aligned uint8 buffer (torch's caching allocator aligns to >= 512 B)."""
    t = torch.empty(max(int(n), 256), dtype=torch.uint8, device=device)
    assert t.data_ptr() % 256 == 0
    return t


class GramState:
    """The one-pass second-moment state of a calibration run (device buffer + layout)."""

    def __init__(self, d: int, n_targets: int, dtype, device, stream=None, d_out: int = 0):
        self.desc = gram_desc(d, n_targets, dtype, d_out)
        self.layout = rf_gram_state_layout(self.desc)
        self.buf = device_bytes(rf_gram_state_bytes(self.desc), device)
        self.d, self.n_targets = d, n_targets
        self.dy = d_out or d
        rf_gram_init(self.desc, self.buf, stream)

    def accumulate(self, X, Ys, stream=None):
        rf_gram_accumulate(self.desc, self.buf, X, Ys, stream=stream)

    # views of the state (plain data as laid out by rf_gram_state_layout)
    def _view(self, off, count, dtype):
        nbytes = count * torch.tensor([], dtype=dtype).element_size()
        return self.buf[off:off + nbytes].view(dtype)

    def n(self):
        return self._view(self.layout["off_n"], 1, torch.int64)

    def S_xx(self):
        return self._view(self.layout["off_S_xx"], self.d * self.d, torch.float32).view(self.d, self.d)

    def S_yx(self):
        return self._view(self.layout["off_S_yx"], self.n_targets * self.dy * self.d,
                          torch.float32).view(self.n_targets, self.dy, self.d)

    def s_x(self):
        return self._view(self.layout["off_s_x"], self.d, torch.float64)

    def s_y(self):
        return self._view(self.layout["off_s_y"], self.n_targets * self.dy, torch.float64).view(self.n_targets, self.dy)

    def s_yy(self):
        return self._view(self.layout["off_s_yy"], self.n_targets * self.dy,
                          torch.float64).view(self.n_targets, self.dy)

    def r2(self, lam: float, mode: int, targets: Sequence[int], W, stream=None) -> torch.Tensor:
        """R^2 of the maps W (rf_solve's fp32 output for ``targets``), read off the state."""
        dev = self.buf.device
        out = torch.empty(len(targets), dtype=torch.float64, device=dev)
        ws = device_bytes(rf_fit_r2_workspace_bytes(self.desc, len(targets)), dev)
        rf_fit_r2(self.desc, self.buf, lam, mode, list(targets), W, out, ws, stream)
        return out

    def solve_pinv(self, lam: float, mode: int, targets: Sequence[int], rel_tol: float = 1e-8, sweeps: int = 15,
                   want_bf16=False, stream=None):
        """The maps by the eigendecomposition pseudo-inverse route (rf_solve_pinv)."""
        dev = self.buf.device
        n_sel = len(targets)
        W = torch.empty(n_sel, self.dy, self.d, dtype=torch.float32, device=dev)
        Wlp = torch.empty(n_sel, self.dy, self.d, dtype=torch.bfloat16, device=dev) if want_bf16 else None
        b = torch.empty(n_sel, self.dy, dtype=torch.float32, device=dev)
        ws = device_bytes(rf_solve_pinv_workspace_bytes(self.desc, n_sel), dev)
        rf_solve_pinv(self.desc, self.buf, lam, mode, rel_tol, sweeps, list(targets), W, Wlp, b, ws, stream)
        return W, Wlp, b

    def solve(self, lam: float, mode: int, targets: Sequence[int], want_f32=True, want_bf16=True, stream=None,
              ws: Optional[torch.Tensor] = None, product: int = RF_PRODUCT_AUTO):
        """Maps for one ridge strength: (W [n_sel, m, d] fp32, W_lp packed bf16, b, info [1])."""
        W, Wlp, b, info, _, _ = self.solve_many([lam], mode, targets, want_f32, want_bf16, stream, ws, product)
        return (None if W is None else W[0], None if Wlp is None else Wlp[0], b[0], info)

    def solve_many(self, lambdas: Sequence[float], mode: int, targets: Sequence[int], want_f32=True, want_bf16=True,
                   stream=None, ws: Optional[torch.Tensor] = None, product: int = RF_PRODUCT_AUTO,
                   want_resid: bool = False):
        """Maps for a batch of ridge strengths from one call (rf_solve): W [n_lambda, n_sel, m, d]
        fp32, W_lp (packed bf16), b [n_lambda, n_sel, m], info [n_lambda], cond [n_lambda] (the
        largest entry of the equilibrated inverse) and, with ``want_resid``, the stationarity
        residual [n_lambda, n_sel] (fp64)."""
        dev = self.buf.device
        n_sel, nl = len(targets), len(lambdas)
        W = torch.empty(nl, n_sel, self.dy, self.d, dtype=torch.float32, device=dev) if want_f32 or want_resid else None
        Wlp = torch.empty(nl, n_sel, self.dy, self.d, dtype=torch.bfloat16, device=dev) if want_bf16 else None
        b = torch.empty(nl, n_sel, self.dy, dtype=torch.float32, device=dev)
        info = torch.empty(nl, dtype=torch.int32, device=dev)
        cond = torch.empty(nl, dtype=torch.float64, device=dev)
        resid = torch.empty(nl, n_sel, dtype=torch.float64, device=dev) if want_resid else None
        if ws is None:
            ws = device_bytes(rf_solve_workspace_bytes(self.desc, n_sel, nl), dev)
        rf_solve(self.desc, self.buf, list(lambdas), mode, list(targets), W, Wlp, b, info, ws, stream,
                 product=product, cond=cond, resid=resid)
        return W, Wlp, b, info, cond, resid


def solve_headwise(state: GramState, lam: float, mode: int, head_dim: int, targets: Sequence[int], stream=None,
                   product: int = RF_PRODUCT_AUTO):
    """Head-wise maps from one state (rf_solve_headwise): W [n_sel, m, d] fp32 (block-diagonal by
    head, zero between heads), b [n_sel, m], info [1]."""
    dev = state.buf.device
    n_sel = len(targets)
    W = torch.empty(n_sel, state.dy, state.d, dtype=torch.float32, device=dev)
    b = torch.empty(n_sel, state.dy, dtype=torch.float32, device=dev)
    info = torch.empty(1, dtype=torch.int32, device=dev)
    ws = device_bytes(rf_solve_workspace_bytes(state.desc, n_sel, 1), dev)
    rf_solve_headwise(state.desc, state.buf, lam, mode, head_dim, list(targets), W, None, b, info, ws, stream,
                      product=product)
    return W, b, info


def greedy_sources(state: GramState, block_width: int, nu: int, lam: float, mode: int,
                   targets: Optional[Sequence[int]] = None, stream=None, return_order: bool = False):
    """Greedy match (KV-Lingo page, section 3.1): for each target, forward selection over the
    column blocks of X (source layers) by the R^2 of the joint ridge fit, all of it read off
    the one accumulated state.  Each step scores every candidate set E + {s} with
    rf_gram_select -> rf_solve -> rf_fit_r2 (a set shared by several targets is solved once
    for all of them) and keeps the best per target (equal scores: the shallower layer).
    A candidate set whose regularised Gram is not positive definite (the solve's pivot
    report, e.g. lambda = 0 with a source layer of constant rows) or whose score is not
    finite ranks last; a step with no valid candidate raises.
    The sub-state, the solve and R^2 workspaces and the maps are allocated once, for the
    largest set (nu blocks), and reused by every candidate; each candidate's scores and pivot
    report stay on the device until the step's candidates are all enqueued, then come back in
    one copy.  The choices are host decisions on the scores; every number comes from the
    library.  Returns the chosen layers per target, ascending; with ``return_order`` also the
    picks in the order they were made."""
    dev = state.buf.device
    n_blocks = state.d // block_width
    targets = list(range(state.n_targets)) if targets is None else list(targets)
    chosen: List[List[int]] = [[] for _ in targets]
    n_t = len(set(targets))
    # buffers for the largest candidate set, reused by all of them
    big = gram_desc(nu * block_width, state.n_targets, state.desc.dtype, state.desc.d_out)
    sub_buf = device_bytes(max(rf_gram_state_bytes(gram_desc(k * block_width, state.n_targets, state.desc.dtype,
                                                             state.desc.d_out)) for k in range(1, nu + 1)), dev)
    solve_ws = device_bytes(max(rf_solve_workspace_bytes(gram_desc(k * block_width, state.n_targets,
                                                                   state.desc.dtype, state.desc.d_out), n_t, 1)
                                for k in range(1, nu + 1)), dev)
    r2_ws = device_bytes(max(rf_fit_r2_workspace_bytes(gram_desc(k * block_width, state.n_targets, state.desc.dtype,
                                                                 state.desc.d_out), n_t) for k in range(1, nu + 1)), dev)
    W_buf = torch.empty(n_t * state.dy * big.d, dtype=torch.float32, device=dev)
    b_buf = torch.empty(n_t * state.dy, dtype=torch.float32, device=dev)
    for _ in range(nu):
        sets: dict = {}
        for ti in range(len(targets)):
            for s in range(n_blocks):
                if s not in chosen[ti]:
                    sets.setdefault(tuple(sorted(chosen[ti] + [s])), []).append(ti)
        keys = list(sets)
        r2_dev = torch.empty(len(keys), n_t, dtype=torch.float64, device=dev)
        info_dev = torch.empty(len(keys), dtype=torch.int32, device=dev)
        tsels = []
        for c, key in enumerate(keys):
            sub_desc = gram_desc(len(key) * block_width, state.n_targets, state.desc.dtype, state.desc.d_out)
            rf_gram_select(state.desc, state.buf, block_width, list(key), sub_desc, sub_buf, stream)
            tsel = sorted(set(targets[ti] for ti in sets[key]))
            tsels.append(tsel)
            W = W_buf[:len(tsel) * state.dy * sub_desc.d]
            rf_solve(sub_desc, sub_buf, lam, mode, tsel, W, None, b_buf[:len(tsel) * state.dy], info_dev[c:c + 1],
                     solve_ws, stream)
            rf_fit_r2(sub_desc, sub_buf, lam, mode, tsel, W, r2_dev[c, :len(tsel)], r2_ws, stream)
        r2_host = r2_dev.cpu().tolist()
        info_host = info_dev.cpu().tolist()
        scores: dict = {}
        for c, key in enumerate(keys):
            ok = info_host[c] == 0
            for t, v in zip(tsels[c], r2_host[c]):
                scores[(key, t)] = v if ok and math.isfinite(v) else None
        for ti, t in enumerate(targets):
            best = None
            for s in range(n_blocks):
                if s in chosen[ti]:
                    continue
                v = scores[(tuple(sorted(chosen[ti] + [s])), t)]
                if v is not None and (best is None or v > best[0]):
                    best = (v, s)
            if best is None:
                raise RuntimeError(f"greedy match: no candidate set of target {t} can be fitted "
                                   f"(every regularised Gram failed its factorisation or scored non-finite)")
            chosen[ti].append(best[1])
    sets = [sorted(c) for c in chosen]
    return (sets, [list(c) for c in chosen]) if return_order else sets


@dataclass
class Cache:
    desc: object
    layout: dict
    k: List[torch.Tensor]
    v: List[torch.Tensor]
    block_table: Optional[torch.Tensor]


def alloc_cache(n_layers: int, n_kv_heads: int, head_dim: int, max_tokens: int, dtype, device,
                paged: bool = False, block_size: int = 16, block_table: Optional[torch.Tensor] = None,
                sentinel: float = float("nan"), n_blocks: Optional[int] = None) -> Cache:
    desc = cache_desc(n_kv_heads, head_dim, max_tokens, RF_LAYOUT_PAGED if paged else RF_LAYOUT_CONTIGUOUS,
                      dtype, block_size)
    if paged and n_blocks is not None:
        desc.max_tokens = n_blocks * block_size
    lay = rf_cache_layout(desc)
    n_el = lay["bytes_per_pool"] // lay["elem_bytes"]
    k = [torch.full((n_el,), sentinel, dtype=dtype, device=device) for _ in range(n_layers)]
    v = [torch.full((n_el,), sentinel, dtype=dtype, device=device) for _ in range(n_layers)]
    return Cache(desc, lay, k, v, block_table)


def gather_rows(cache: Cache, pool: torch.Tensor, t0: int, t1: int) -> torch.Tensor:
    """Rows [t0, t1) of one pool as [t1 - t0, H, d_h] (index arithmetic only)."""
    H, dh = cache.desc.n_kv_heads, cache.desc.head_dim
    if cache.desc.layout == RF_LAYOUT_CONTIGUOUS:
        return pool.view(-1, H, dh)[t0:t1]
    bs = cache.desc.block_size
    t = torch.arange(t0, t1, device=pool.device)
    phys = cache.block_table.long()[t // bs]
    blocks = pool.view(-1, H, bs, dh)
    return blocks[phys, :, t % bs, :]


def pack_weights(W: torch.Tensor, rope_head_dim: int = 0, stream=None) -> torch.Tensor:
    """A packed bf16 copy (rf_pack_weights) of a bf16 or fp32 [rows, cols] weight matrix."""
    out = torch.empty(W.shape[0], W.shape[1], dtype=torch.bfloat16, device=W.device)
    rf_pack_weights(W, out, rope_head_dim, stream)
    return out


def quantize_map(W: torch.Tensor, stream=None):
    """(codes, scales) of rf_quantize_map for a [rows, cols] map (fp32, or upcast to it): int8
    codes in packed order and [rows] fp32 row scales."""
    W32 = W.float().contiguous()
    q = torch.empty(W.shape[0], W.shape[1], dtype=torch.int8, device=W.device)
    s = torch.empty(W.shape[0], dtype=torch.float32, device=W.device)
    rf_quantize_map(W32, q, s, stream)
    return q, s


def fill_weights(d: int, n_kv_heads: int, head_dim: int, rms_eps: float, dtype, W_map, b_map, gamma, W_k, W_v,
                 stream=None, k_norm=None, k_norm_eps: float = 1e-6, int8_maps: bool = False) -> FillWeights:
    """FillWeights from row-major weights: bf16 maps and projections are packed first (the
    fp32 path reads them as they are); with ``int8_maps`` (bf16 only) the maps become
    weight-only int8 codes with row scales (rf_quantize_map)."""
    scales = None
    if dtype == torch.bfloat16:
        if int8_maps:
            qs = [quantize_map(W, stream) for W in W_map]
            W_map, scales = [q for q, _ in qs], [s for _, s in qs]
        else:
            W_map = [pack_weights(W, 0, stream) for W in W_map]
        W_k = [pack_weights(W, head_dim, stream) for W in W_k]
        W_v = [pack_weights(W, head_dim, stream) for W in W_v]
    elif int8_maps:
        raise ValueError("int8 maps need bf16 weights")
    return FillWeights(d, n_kv_heads, head_dim, rms_eps, dtype, list(W_map), list(b_map), list(gamma), list(W_k),
                       list(W_v), None if k_norm is None else list(k_norm), k_norm_eps, scales)


class Filler:
    """Holds the per-layer weights, a RoPE table and a workspace; fills token ranges."""

    def __init__(self, weights: FillWeights, rope_base: float, max_pos: int, max_rows: int, device,
                 ws_slots: int = 1, stream=None):
        self.w = weights
        self.rope_len = max_pos
        self.rope = torch.empty(max_pos, weights.head_dim, dtype=torch.float32, device=device)
        rf_rope_table(rope_base, weights.head_dim, max_pos, self.rope, stream)
        self.ws = device_bytes(rf_fill_workspace_bytes(weights, max_rows) * max(1, ws_slots), device)

    def fill(self, X, t0: int, t1: int, pos0: int, cache: Cache, stream=None):
        rf_fill(self.w, X, t0, t1, pos0, cache.desc, cache.k, cache.v, cache.block_table, self.rope,
                self.rope_len, self.ws, stream)


def compose_weights(weights: FillWeights, stream=None, slots: int = 8) -> ComposedFillWeights:
    """The composed weights (rf_fill_compose) of every layer of a bf16 FillWeights, in fresh
    device buffers (``slots`` layers per product launch)."""
    dev = weights.W_map[0].device
    L, d, kvw = len(weights.W_map), weights.d, weights.n_kv_heads * weights.head_dim
    T = [torch.empty(d, d, dtype=torch.bfloat16, device=dev) for _ in range(L)]
    q = [torch.empty(2 * d + 4, dtype=torch.float32, device=dev) for _ in range(L)]
    Mk = [torch.empty(kvw, d, dtype=torch.bfloat16, device=dev) for _ in range(L)]
    Mv = [torch.empty(kvw, d, dtype=torch.bfloat16, device=dev) for _ in range(L)]
    ck = [torch.empty(kvw, dtype=torch.float32, device=dev) for _ in range(L)]
    cv = [torch.empty(kvw, dtype=torch.float32, device=dev) for _ in range(L)]
    out = ComposedFillWeights(d, weights.n_kv_heads, weights.head_dim, weights.rms_eps, T, q, Mk, Mv, ck, cv,
                              weights.k_norm, weights.k_norm_eps, weights.rope_base)
    ws = device_bytes(rf_fill_compose_workspace_bytes(weights) * max(1, min(slots, L)), dev)
    rf_fill_compose(weights, out, ws, stream)
    return out


class ComposedFiller:
    """Composed weights (rf_fill_compose), a RoPE table and a workspace; fills token ranges
    with rf_fill_composed."""

    def __init__(self, weights: FillWeights, rope_base: float, max_pos: int, max_rows: int, device, ws_slots: int = 32,
                 stream=None, composed: Optional[ComposedFillWeights] = None):
        self.w = composed if composed is not None else compose_weights(weights, stream)
        self.rope_len = max_pos
        self.rope = torch.empty(max_pos, weights.head_dim, dtype=torch.float32, device=device)
        rf_rope_table(rope_base, weights.head_dim, max_pos, self.rope, stream)
        self.ws = device_bytes(rf_fill_composed_workspace_bytes(self.w, max_rows) * max(1, ws_slots), device)

    def fill(self, X, t0: int, t1: int, pos0: int, cache: Cache, stream=None):
        rf_fill_composed(self.w, X, t0, t1, pos0, cache.desc, cache.k, cache.v, cache.block_table, self.rope,
                         self.rope_len, self.ws, stream)


class StreamedFiller(Filler):
    """A Filler whose maps stay in page-locked host memory and stream through a device ring
    (rf_fill_streamed); the workspace holds ``layers_per_slot`` layer slots."""

    def __init__(self, weights: FillWeights, rope_base: float, max_pos: int, max_rows: int, device,
                 ring_slots: int = 2, layers_per_slot: int = 1, stream=None, rows_per_fill: int = 0):
        """rows_per_fill: tokens per fill step inside each layer chunk (0: a call's whole range,
        which must then fit ``max_rows``); the workspace covers one step."""
        step_rows = rows_per_fill if rows_per_fill > 0 else max_rows
        super().__init__(weights, rope_base, max_pos, step_rows, device, ws_slots=layers_per_slot, stream=stream)
        self.ring_slots, self.layers_per_slot, self.rows_per_fill = ring_slots, layers_per_slot, rows_per_fill
        self.ring = device_bytes(rf_fill_streamed_ring_bytes(weights, ring_slots, layers_per_slot), device)
        self.copy_stream = torch.cuda.Stream(device=device)

    def fill(self, X, t0: int, t1: int, pos0: int, cache: Cache, stream=None):
        rf_fill_streamed(self.w, X, t0, t1, pos0, cache.desc, cache.k, cache.v, cache.block_table, self.rope,
                         self.rope_len, self.ws, self.ring, self.ring_slots, self.layers_per_slot,
                         stream if stream is not None else torch.cuda.current_stream(), self.copy_stream,
                         rows_per_fill=self.rows_per_fill)


def pinned_copy(t: torch.Tensor) -> torch.Tensor:
    """A page-locked host copy of a tensor (allocated pinned, then filled)."""
    out = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
    out.copy_(t)
    return out


def translate_weights(d_in: int, n_kv_heads: int, head_dim: int, dtype, T_k, T_v, b_k=None, b_v=None,
                      stream=None, headwise: bool = False, k_norm=None, k_norm_eps: float = 1e-6) -> TranslateWeights:
    """TranslateWeights from row-major [kv_width, d_in] maps: for bf16 they are packed first
    (fp32 maps are rounded to bf16 by the packing); the fp32 path reads them as they are."""
    if dtype == torch.bfloat16:
        T_k = [pack_weights(T, head_dim, stream) for T in T_k]
        T_v = [pack_weights(T, head_dim, stream) for T in T_v]
    return TranslateWeights(d_in, n_kv_heads, head_dim, dtype, list(T_k), list(T_v),
                            None if b_k is None else list(b_k), None if b_v is None else list(b_v), headwise,
                            None if k_norm is None else list(k_norm), k_norm_eps)


class Translator:
    """Holds the per-target-layer translator maps and a RoPE table; translates token ranges.
    ``rope_base=None``: no table, keys stored unrotated (post-RoPE translators)."""

    def __init__(self, weights: TranslateWeights, rope_base, max_pos: int, device, stream=None):
        self.w = weights
        self.rope_len = max_pos if rope_base is not None else 0
        self.rope = None
        if rope_base is not None:
            self.rope = torch.empty(max_pos, weights.head_dim, dtype=torch.float32, device=device)
            rf_rope_table(rope_base, weights.head_dim, max_pos, self.rope, stream)

    def translate(self, src_k: Sequence, src_v: Sequence, ld_src: int, t0: int, t1: int, pos0: int, cache: Cache,
                  stream=None):
        rf_translate(self.w, src_k, src_v, ld_src, t0, t1, pos0, cache.desc, cache.k, cache.v, cache.block_table,
                     self.rope, self.rope_len, stream)
