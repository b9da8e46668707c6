"""Seeded synthetic workloads for the ridge fit and the late-layer cache fill.

This module only draws random inputs of the shapes and laws the workloads name.  It holds
none of the method's arithmetic (no Gram, solve, norm, projection or rotation), so the
oracle and the HIP path can both consume what it produces without sharing any of the
method's code.

Every tensor is drawn from a ``torch.Generator`` seeded by a hash of
``(config seed, tensor name, layer, chunk)``, so any chunk or layer can be regenerated on
its own, on the CPU or directly on the GPU.  Values are rounded to the configuration's
storage dtype (fp32 or bf16) before they are handed to either side.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field, replace
from typing import Optional, Sequence

import torch


@dataclass(frozen=True)
class Config:
    """One workload: the model shape, the calibration set and the prompt to fill."""

    name: str
    d: int                      # hidden width
    n_layers: int               # layers of the model
    split: int                  # first late layer; layers [split, n_layers) are filled
    n_kv_heads: int
    head_dim: int
    rms_eps: float
    rope_base: float
    dtype: str                  # storage dtype of X, Y, maps, K/V weights and cache: 'f32' | 'bf16'
    calib_rows: int             # calibration rows N (0: no fit in this workload)
    calib_chunk: int            # rows per accumulate call
    lambdas: tuple              # ridge strengths
    prompt_tokens: int          # T
    fill_t0: int                # filled token range [fill_t0, fill_t1)
    fill_t1: int
    fill_chunk: int             # tokens per fill call
    paged: bool
    block_size: int
    x_law: str                  # 'gauss' | 'lognormal_scales' | 'outliers'
    y_law: str                  # 'planted_dense' | 'identity_perm'
    fill_maps: str              # 'fitted' | 'random'
    seed: int
    n_targets_override: int = 0  # fit-only workloads: number of target layers

    @property
    def filled_layers(self) -> list:
        return list(range(self.split, self.n_layers))

    @property
    def n_targets(self) -> int:
        return self.n_targets_override or (self.n_layers - self.split)

    @property
    def kv_width(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def fill_tokens(self) -> int:
        return self.fill_t1 - self.fill_t0

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def fill_flop_per_token_layer(self) -> int:
        """Algorithmic multiply-add work of one filled (token, layer): map GEMM plus K/V GEMM."""
        return 2 * self.d * (self.d + 2 * self.kv_width)

    def fit_flop_per_row(self) -> int:
        """Algorithmic Gram work per calibration row: upper triangle of X^T X plus X^T Y."""
        return self.d * (self.d + 1) + 2 * self.n_targets * self.d * self.d


C1 = Config(name="tiny-fp32-d256", d=256, n_layers=8, split=4, n_kv_heads=4, head_dim=64,
            rms_eps=1e-6, rope_base=1e4, dtype="f32", calib_rows=4096, calib_chunk=4096,
            lambdas=(1e-2,), prompt_tokens=512, fill_t0=0, fill_t1=512, fill_chunk=512,
            paged=False, block_size=16, x_law="gauss", y_law="planted_dense",
            fill_maps="fitted", seed=1001)

C2 = Config(name="llama8b-shaped-d4096-T16384", d=4096, n_layers=32, split=16, n_kv_heads=8,
            head_dim=128, rms_eps=1e-6, rope_base=5e5, dtype="bf16", calib_rows=65536,
            calib_chunk=32768, lambdas=(1e-1,), prompt_tokens=16384, fill_t0=0, fill_t1=16384,
            fill_chunk=16384, paged=False, block_size=16, x_law="lognormal_scales",
            y_law="identity_perm", fill_maps="fitted", seed=1002)

C3 = Config(name="27b-shaped-d5120-T32768", d=5120, n_layers=64, split=16, n_kv_heads=8,
            head_dim=128, rms_eps=1e-6, rope_base=5e5, dtype="bf16", calib_rows=0,
            calib_chunk=0, lambdas=(), prompt_tokens=32768, fill_t0=2048, fill_t1=28672,
            fill_chunk=28672 - 2048, paged=False, block_size=16, x_law="gauss",
            y_law="identity_perm", fill_maps="random", seed=1003)

C4 = Config(name="fit-heavy-d4096-N262144", d=4096, n_layers=32, split=16, n_kv_heads=8,
            head_dim=128, rms_eps=1e-6, rope_base=5e5, dtype="bf16", calib_rows=262144,
            calib_chunk=8192, lambdas=(1e-3, 1e-1, 10.0), prompt_tokens=0, fill_t0=0,
            fill_t1=0, fill_chunk=0, paged=False, block_size=16, x_law="lognormal_scales",
            y_law="identity_perm", fill_maps="fitted", seed=1004, n_targets_override=16)

C5 = Config(name="long-context-d4096-T131072-paged", d=4096, n_layers=32, split=16,
            n_kv_heads=8, head_dim=128, rms_eps=1e-6, rope_base=5e5, dtype="bf16",
            calib_rows=0, calib_chunk=0, lambdas=(), prompt_tokens=131072, fill_t0=0,
            fill_t1=131072 - 4096, fill_chunk=8192, paged=True, block_size=16,
            x_law="outliers", y_law="identity_perm", fill_maps="random", seed=1005)

CONFIGS = {"C1": C1, "C2": C2, "C3": C3, "C4": C4, "C5": C5}


def scaled(cfg: Config, **kw) -> Config:
    """A copy of ``cfg`` with some fields changed (smaller parity cases of the same law)."""
    return replace(cfg, **kw)


# ----------------------------------------------------------------------------------------
# seeding
# ----------------------------------------------------------------------------------------

def _seed(cfg_seed: int, *key) -> int:
    h = hashlib.sha256(repr((cfg_seed,) + tuple(key)).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def generator(cfg_seed: int, *key, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(cfg_seed, *key))
    return g


def _randn(shape, cfg_seed, *key, device="cpu"):
    g = generator(cfg_seed, *key, device=device)
    return torch.randn(*shape, generator=g, device=device, dtype=torch.float32)


def _store(t: torch.Tensor, cfg: Config) -> torch.Tensor:
    return t.to(cfg.torch_dtype).contiguous()


# ----------------------------------------------------------------------------------------
# hidden states
# ----------------------------------------------------------------------------------------

def channel_scales(cfg: Config, device="cpu") -> torch.Tensor:
    """Per-channel scale of the split-layer state: s_j ~ LogNormal(0, 0.5), or the
    outlier law (1 % of channels, a seeded choice, scaled by 20), or all ones."""
    if cfg.x_law == "lognormal_scales":
        return torch.exp(0.5 * _randn((cfg.d,), cfg.seed, "scale", device=device))
    s = torch.ones(cfg.d, device=device)
    if cfg.x_law == "outliers":
        n_out = max(1, round(0.01 * cfg.d))
        g = generator(cfg.seed, "outlier_channels", device="cpu")
        idx = torch.randperm(cfg.d, generator=g)[:n_out].to(device)
        s[idx] = 20.0
    return s


def hidden_states(cfg: Config, rows: int, stream: str, chunk: int = 0, device="cpu",
                  row_offset: int = 0) -> torch.Tensor:
    """Rows of the split-layer state X, [rows, d] in the storage dtype.

    ``stream`` names an independent draw ('calib' or 'prompt'); ``chunk`` selects a block
    of rows within it so chunks can be drawn one at a time."""
    z = _randn((rows, cfg.d), cfg.seed, "X", stream, chunk, row_offset, device=device)
    return _store(z * channel_scales(cfg, device=device), cfg)


def low_rank_states(cfg: Config, rows: int, stream: str, chunk: int = 0, device="cpu", rank: int = 64,
                    sigma: float = 0.2, n_dup: int = 8, dup_noise: float = 0.2) -> torch.Tensor:
    """Rows of an anisotropic split-layer state of low effective rank with near-duplicate
    channels, [rows, d] in the storage dtype: the shape of trained caches in the KV-Lingo
    page's rank table (appendix B.2, Table 3: effective rank far below the width, a few
    directions carrying most of the variance).
        X = (F M + sigma Z) * s
    F [rows, rank] ~ N(0, 1) per chunk; M [rank, d] a fixed seeded mixing whose row i has
    scale 3 exp(-4 i / rank) / sqrt(rank); Z ~ N(0, 1); channel 2k + 1 is then channel 2k plus
    dup_noise N(0, 1) for k < n_dup; s the per-channel log-normal scales."""
    F = _randn((rows, rank), cfg.seed, "lowrank-F", stream, chunk, device=device)
    decay = 3.0 * torch.exp(-4.0 * torch.arange(rank, dtype=torch.float32, device=device) / rank) / rank ** 0.5
    M = _randn((rank, cfg.d), cfg.seed, "lowrank-M", device=device) * decay[:, None]
    X = F @ M + sigma * _randn((rows, cfg.d), cfg.seed, "lowrank-Z", stream, chunk, device=device)
    D = _randn((rows, n_dup), cfg.seed, "lowrank-dup", stream, chunk, device=device)
    for k in range(n_dup):
        X[:, 2 * k + 1] = X[:, 2 * k] + dup_noise * D[:, k]
    s = torch.exp(0.5 * _randn((cfg.d,), cfg.seed, "lowrank-scale", device=device))
    return _store(X * s, cfg)


def planted_map(cfg: Config, layer: int, device="cpu") -> torch.Tensor:
    """Dense planted map A_l ~ N(0, 1/d), [d_in, d_out] (x-times-matrix convention)."""
    return _randn((cfg.d, cfg.d), cfg.seed, "A", layer, device=device) / cfg.d ** 0.5


def signed_permutation(cfg: Config, layer: int):
    """(perm, sign) of the signed permutation P_l: (X P_l)[:, j] = sign[j] * X[:, perm[j]]."""
    g = generator(cfg.seed, "P", layer, device="cpu")
    perm = torch.randperm(cfg.d, generator=g)
    sign = torch.randint(0, 2, (cfg.d,), generator=g).float() * 2 - 1
    return perm, sign


def late_layer_inputs(cfg: Config, X: torch.Tensor, layer: int, chunk: int = 0,
                      row_offset: int = 0) -> torch.Tensor:
    """Synthetic capture Y_l of a late layer's input for calibration rows X.

    planted_dense : Y = X A_l + 0.1 E
    identity_perm : Y = X (I + 0.02 P_l) + 0.1 E, P_l a signed permutation
    E ~ N(0, 1) is drawn per (layer, chunk).  This is the data law of the workload, not a
    step of the method."""
    device = X.device
    Xf = X.float()
    E = _randn(tuple(X.shape), cfg.seed, "E", layer, chunk, row_offset, device=device)
    if cfg.y_law == "planted_dense":
        Y = Xf @ planted_map(cfg, layer, device=device) + 0.1 * E
    else:
        perm, sign = signed_permutation(cfg, layer)
        Y = Xf + 0.02 * Xf[:, perm.to(device)] * sign.to(device) + 0.1 * E
    return _store(Y, cfg)


# ----------------------------------------------------------------------------------------
# fill weights
# ----------------------------------------------------------------------------------------

@dataclass
class LayerWeights:
    """Stored weights of one filled layer, in the library's layouts.

    W_map : [d_out, d_in]  map, out-feature major (h = x W_map^T + b_map)
    b_map : [d] fp32
    gamma : [d] fp32       RMSNorm weight
    W_k   : [H_kv*d_h, d]  K projection, out-feature major (k = u W_k^T), head-major rows
    W_v   : [H_kv*d_h, d]
    """

    W_map: torch.Tensor
    b_map: torch.Tensor
    gamma: torch.Tensor
    W_k: torch.Tensor
    W_v: torch.Tensor


def kv_weights(cfg: Config, layer: int, device="cpu"):
    Wk = 0.02 * _randn((cfg.kv_width, cfg.d), cfg.seed, "Wk", layer, device=device)
    Wv = 0.02 * _randn((cfg.kv_width, cfg.d), cfg.seed, "Wv", layer, device=device)
    gamma = 1.0 + 0.02 * _randn((cfg.d,), cfg.seed, "gamma", layer, device=device)
    return _store(Wk, cfg), _store(Wv, cfg), gamma.float().contiguous()


def key_norm_weights(cfg, layer: int, device="cpu") -> torch.Tensor:
    """Per-head key norm weights gamma_k [head_dim] = 1 + N(0, 0.1^2), fp32 (for models that
    normalise keys per head)."""
    return (1.0 + 0.1 * _randn((cfg.head_dim,), cfg.seed, "gk", layer, device=device)).contiguous()


def random_map(cfg: Config, layer: int, device="cpu"):
    """Random-init map centred on the identity fill: W = I + N(0, 0.02^2), b ~ N(0, 0.02^2)."""
    W = 0.02 * _randn((cfg.d, cfg.d), cfg.seed, "Wmap", layer, device=device)
    W += torch.eye(cfg.d, device=device)
    b = 0.02 * _randn((cfg.d,), cfg.seed, "bmap", layer, device=device)
    return _store(W, cfg), b.float().contiguous()


def law_map(cfg: Config, layer: int, device="cpu"):
    """A map of the law the fit recovers for ``identity_perm`` data: I + 0.02 P_l plus a
    small perturbation, stored out-feature major.  Used where a fill needs maps of the
    fitted law without running a fit."""
    perm, sign = signed_permutation(cfg, layer)
    W = torch.eye(cfg.d, device=device)
    # (x (I + 0.02 P))_j = x_j + 0.02 sign_j x_perm[j]  ->  out-major row j has 0.02 sign_j at perm[j]
    W[torch.arange(cfg.d, device=device), perm.to(device)] += 0.02 * sign.to(device)
    W += 1e-3 * _randn((cfg.d, cfg.d), cfg.seed, "Wlaw", layer, device=device)
    b = 1e-3 * _randn((cfg.d,), cfg.seed, "blaw", layer, device=device)
    return _store(W, cfg), b.float().contiguous()


def layer_weights(cfg: Config, layer: int, device="cpu", maps: Optional[str] = None) -> LayerWeights:
    maps = maps or cfg.fill_maps
    if maps == "random":
        W, b = random_map(cfg, layer, device)
    elif maps == "identity":
        W = _store(torch.eye(cfg.d, device=device), cfg)
        b = torch.zeros(cfg.d, device=device)
    else:
        W, b = law_map(cfg, layer, device)
    Wk, Wv, gamma = kv_weights(cfg, layer, device)
    return LayerWeights(W, b, gamma, Wk, Wv)


def block_table(cfg: Config, n_tokens: int, device="cpu", extra_blocks: int = 3) -> torch.Tensor:
    """Shuffled logical->physical block table for a paged cache with a few spare blocks."""
    n_logical = -(-n_tokens // cfg.block_size)
    g = generator(cfg.seed, "block_table", device="cpu")
    phys = torch.randperm(n_logical + extra_blocks, generator=g)[:n_logical]
    return phys.to(torch.int32).to(device)


# ----------------------------------------------------------------------------------------
# KV-cache translation workloads (token-wise linear translators between two models' caches)
# ----------------------------------------------------------------------------------------

@dataclass(frozen=True)
class TranslateConfig:
    """One translation workload: a source cache of n_src layers, a target of n_tgt layers,
    each target layer reading nu source layers (relative-depth bands)."""

    name: str
    n_src: int
    src_kv_heads: int
    src_head_dim: int
    n_tgt: int
    n_kv_heads: int
    head_dim: int
    nu: int
    rope_base: float
    dtype: str
    tokens: int                 # prompt tokens held by the source cache
    t0: int                     # translated token range [t0, t1)
    t1: int
    paged: bool
    block_size: int
    maps: str                   # 'dense' (head-mixing) | 'headwise' (block-diagonal)
    bias: bool
    seed: int

    @property
    def d_src(self) -> int:
        return self.src_kv_heads * self.src_head_dim

    @property
    def d_in(self) -> int:
        return self.nu * self.d_src

    @property
    def kv_width(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def flop_per_token_layer(self) -> int:
        """Algorithmic work of one translated (token, target layer): K and V products (the
        head blocks only, for head-wise maps)."""
        if self.maps == "headwise":
            return 2 * 2 * self.nu * self.n_kv_heads * self.head_dim * self.src_head_dim
        return 2 * 2 * self.d_in * self.kv_width


# The KV-Lingo page's cross-layer pairs: caches of 28 and 36 layers, 8 KV heads x 128 on both
# sides, head-mixing maps reading 2 source layers (section 4, cross-layer pairs).
TR_BENCH = TranslateConfig(name="kv-translate-28to36-kv8x128-nu2-T16384", n_src=28, src_kv_heads=8,
                           src_head_dim=128, n_tgt=36, n_kv_heads=8, head_dim=128, nu=2, rope_base=5e5,
                           dtype="bf16", tokens=16384, t0=0, t1=16384, paged=False, block_size=16,
                           maps="dense", bias=False, seed=1006)


def _tstore(t: torch.Tensor, cfg: TranslateConfig) -> torch.Tensor:
    return t.to(cfg.torch_dtype).contiguous()


def source_cache(cfg: TranslateConfig, rows: int, device="cpu", row_offset: int = 0):
    """Source keys (before rotation) and values of ``rows`` tokens, [rows, n_src, d_src] each
    (token-major, source layers side by side).  Keys carry per-channel scales
    ~ LogNormal(0, 0.5) per layer (key channels differ in magnitude); values are N(0, 1)."""
    ks = torch.exp(0.5 * _randn((cfg.n_src, cfg.d_src), cfg.seed, "kscale", device=device))
    K = _randn((rows, cfg.n_src, cfg.d_src), cfg.seed, "srcK", row_offset, device=device) * ks
    V = _randn((rows, cfg.n_src, cfg.d_src), cfg.seed, "srcV", row_offset, device=device)
    return _tstore(K, cfg), _tstore(V, cfg)


def translator_maps(cfg: TranslateConfig, layer: int, device="cpu"):
    """(T_k, T_v, b_k, b_v) of one target layer: T [kv_width, d_in] out-feature major with
    entries ~ N(0, 1/d_in) (zero outside the diagonal head blocks of each source layer for
    'headwise'); b ~ N(0, 0.1^2) or None."""
    out = []
    for side in ("Tk", "Tv"):
        T = _randn((cfg.kv_width, cfg.d_in), cfg.seed, side, layer, device=device) / cfg.d_in ** 0.5
        if cfg.maps == "headwise":
            if cfg.src_kv_heads != cfg.n_kv_heads:
                raise ValueError("head-wise maps need as many source as target heads")
            oh = torch.arange(cfg.kv_width, device=device) // cfg.head_dim
            ih = (torch.arange(cfg.d_in, device=device) % cfg.d_src) // cfg.src_head_dim
            T = T * (oh[:, None] == ih[None, :])
        out.append(_tstore(T, cfg))
    bk = bv = None
    if cfg.bias:
        bk = (0.1 * _randn((cfg.kv_width,), cfg.seed, "bk", layer, device=device)).contiguous()
        bv = (0.1 * _randn((cfg.kv_width,), cfg.seed, "bv", layer, device=device)).contiguous()
    return out[0], out[1], bk, bv


def translator_calibration(cfg: TranslateConfig, layer: int, src_rows: torch.Tensor, side: str):
    """Synthetic target cache rows for a closed-form translator fit: Y = S A + 0.1 E with a
    planted A ~ N(0, 1/d_in) [d_in, kv_width] (x-times-matrix) and E ~ N(0, 1); for head-wise
    configurations A links only the same head of every source layer and the target.  The data
    law of the fit workload, not a step of the method."""
    device = src_rows.device
    A = _randn((cfg.d_in, cfg.kv_width), cfg.seed, "Acal", side, layer, device=device) / cfg.d_in ** 0.5
    if cfg.maps == "headwise":
        hi = (torch.arange(cfg.d_in, device=device) % cfg.kv_width) // cfg.head_dim
        ho = torch.arange(cfg.kv_width, device=device) // cfg.head_dim
        A = A * (hi[:, None] == ho[None, :])
    E = _randn((src_rows.shape[0], cfg.kv_width), cfg.seed, "Ecal", side, layer, device=device)
    return _tstore(src_rows.float() @ A + 0.1 * E, cfg)


def translate_block_table(cfg: TranslateConfig, n_tokens: int, device="cpu", extra_blocks: int = 3) -> torch.Tensor:
    n_logical = -(-n_tokens // cfg.block_size)
    g = generator(cfg.seed, "block_table", device="cpu")
    phys = torch.randperm(n_logical + extra_blocks, generator=g)[:n_logical]
    return phys.to(torch.int32).to(device)


# ----------------------------------------------------------------------------------------
# Gated DeltaNet inputs (keys, values, gates, write strengths of a linear-attention layer)
# ----------------------------------------------------------------------------------------

def gdn_inputs(seed: int, layer: int, tokens: int, n_heads: int, d_k: int, d_v: int, dtype=torch.bfloat16,
               device="cpu", row_offset: int = 0):
    """Synthetic per-token inputs of one Gated DeltaNet layer's state update: keys and values
    N(0, 1) [tokens, n_heads * d], stored in ``dtype``; log decays g = -softplus(z) a_h with
    z ~ N(0, 1) and a per-head rate a_h ~ U(0.02, 0.5) (per-token decays around 0.7-0.99);
    write strengths beta = sigmoid(N(0, 1)).  Both fp32 [tokens, n_heads].  Drawn in blocks
    keyed by ``row_offset`` so a prompt can be drawn in chunks."""
    K = _randn((tokens, n_heads * d_k), seed, "gdn-k", layer, row_offset, device=device).to(dtype)
    V = _randn((tokens, n_heads * d_v), seed, "gdn-v", layer, row_offset, device=device).to(dtype)
    g_rate = 0.02 + 0.48 * torch.rand(n_heads, generator=generator(seed, "gdn-rate", layer), device="cpu")
    z = _randn((tokens, n_heads), seed, "gdn-g", layer, row_offset, device=device)
    g = -torch.nn.functional.softplus(z) * g_rate.to(device)
    beta = torch.sigmoid(_randn((tokens, n_heads), seed, "gdn-b", layer, row_offset, device=device))
    return K.contiguous(), V.contiguous(), g.contiguous(), beta.contiguous()
