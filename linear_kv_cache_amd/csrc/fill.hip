// Late-layer cache fill (RidgeFill project page, "Method" steps 2-4 and Figure 2(b)).
//
// Per group of layers, two MFMA GEMM launches:
//   map  : h = x W_map^T + b over [tokens x d]; the epilogue adds the bias, forms per-token
//          partial sums of h^2 over its 256 features (fixed order, no atomics), multiplies by
//          gamma and stores u' = h * gamma in the workspace (storage dtype).
//   kv   : [k | v] = u' [W_k | W_v]^T over [tokens x 2*H*d_h]; the epilogue finishes the
//          RMSNorm with r = 1/sqrt(sum of the partials / d + eps) (u W^T = r * (u' W^T)),
//          rotates K pairs (i, i + d_h/2) by their token's position (KV-Lingo page, sec. 3.1,
//          pre-norm storing) and stores K and V rows into the layer's pools.
// MFMA operands: A = weight rows (features), B = token rows, so each lane's accumulators
// hold 4 consecutive features of one token.  bf16 weights arrive packed in fragment order
// (rf_pack_weights) and go straight to registers; K/V rows are packed in rotate-half pairs so
// a head's RoPE partners sit in the same lane and register, one block apart.  The map may be
// weight-only int8 codes (rf_quantize_map), widened to bf16 in registers.  The bf16 fills run
// the K/V product on 512-feature x 128-token tiles (k_fill_kv4) when the K and V halves are
// whole such tiles, on 256 x 256 tiles (k_fill_kv) otherwise.  The composed fill
// (rf_fill_composed) replaces the map launch by the quadratic form of the RMS (k_fill_norm)
// and runs the K/V product on the prompt states with the composed weights.
#include <math.h>

#include <mutex>
#include <string>
#include <vector>

#include "rf_internal.h"
#include "rf_mfma.h"
#include "rf_pipe.h"
#include "rf_pipe4.h"

namespace rf {

constexpr int kMaxGroup = 32;
constexpr int kFT = 256;  // features per tile
constexpr int kTT = 256;  // tokens per tile

struct MapArgs {
    const void* X;
    int64_t ldx;
    int64_t rows;
    int32_t d;
    int32_t n_ps;            // partial sums per token = d / kFT
    int32_t tok_tiles;       // ceil(rows / kTT)
    void* H;                 // workspace rows [rows][d] per layer slot
    int64_t h_slot;          // elements per layer slot
    float* psum;             // [rows][n_ps] per layer slot
    int64_t ps_slot;
    const void* W[kMaxGroup];
    const float* bias[kMaxGroup];
    const float* gamma[kMaxGroup];
    const float* scale[kMaxGroup];   // Q8: the map rows' scales (W = diag(scale) codes)
};

struct KVArgs {
    const float* psum;
    int64_t ps_slot;
    int32_t n_ps;
    int32_t d;
    int32_t kvw;             // n_kv_heads * head_dim
    int32_t tok_tiles;       // ceil(rows / kTT)
    float eps;
    int64_t rows;
    int64_t t0;
    int64_t pos0;
    const float* rope;       // [pos][head_dim/2][2]
    int32_t paged;
    int32_t block_size;
    int64_t stride_block, stride_head, stride_token;
    int64_t n_blocks;
    const int32_t* block_table;
    int64_t n_table_blocks;
    int64_t ld_in;           // row stride of the product's token operand
    const void* in_k[kMaxGroup];  // token rows feeding the K (in_k) and V (in_v) feature tiles
    const void* in_v[kMaxGroup];
    const float* bk[kMaxGroup];   // per-feature intercepts (translators only)
    const float* bv[kMaxGroup];
    const float* kn[kMaxGroup];   // per-head key norm weights [head_dim] (KN only)
    const float* qb[kMaxGroup];   // NORM: the constant added to each token's sum of squares, or null
    float kn_eps;
    const void* Wk[kMaxGroup];
    const void* Wv[kMaxGroup];
    void* kc[kMaxGroup];
    void* vc[kMaxGroup];
};

template <typename T>
__device__ inline void store4(T* p, float a, float b, float c, float e);
template <>
__device__ inline void store4<bf16_t>(bf16_t* p, float a, float b, float c, float e) {
    *(u32x2*)p = u32x2{pack_bf16x2(a, b), pack_bf16x2(c, e)};
}
template <>
__device__ inline void store4<float>(float* p, float a, float b, float c, float e) {
    *(f32x4*)p = f32x4{a, b, c, e};
}

// The bf16 instantiation runs the software-pipelined core; fp32 runs the plain tile loop.
template <typename T> struct FillCore { using G = TileGemm<T, kFT, kTT, false, false>; };
template <> struct FillCore<bf16_t> { using G = PipeGemm; };
// bf16 weights come pre-packed in fragment order and skip LDS (K/V rows grouped by RoPE pairs).
template <typename T> struct MapCore { using G = typename FillCore<T>::G; };
template <> struct MapCore<bf16_t> { using G = PackedAGemm; };
template <typename T> using KVCore = MapCore<T>;

// Tile of this work-group: layer slot g, feature tile mt, token tile tt.  The grid is 1-D over
// (layer, feature tile, token tile), renumbered so that each XCD works on a compact block of
// 4 feature tiles x 8 token tiles at a time (shared weight and token rows in its L2).
__device__ inline void fill_tile(int n_feat, int n_tok, int& g, int& mt, int& tt) {
    const int per_layer = n_feat * n_tok;
    const int v = xcd_order((int)blockIdx.x, (int)gridDim.x);
    g = v / per_layer;
    grouped_tile(v - g * per_layer, n_feat, n_tok, 4, mt, tt);
}

template <typename G>
__device__ inline void fill_gemm(G& gm, char* lds, const void* A, int64_t lda, int64_t va, const void* B, int64_t ldb,
                                 int64_t vb, int nk) {
    gm.run(lds, Operand{A, lda, va}, Operand{B, ldb, vb}, nk);
}
__device__ inline void fill_gemm(PipeGemm& gm, char* lds, const void* A, int64_t lda, int64_t va, const void* B,
                                 int64_t ldb, int64_t vb, int nk) {
    gm.run(lds, PipeOperand{A, lda, va}, PipeOperand{B, ldb, vb}, nk);
}
__device__ inline void fill_gemm(PackedAGemm& gm, char* lds, const void* A, int64_t lda, int64_t va, const void* B,
                                 int64_t ldb, int64_t vb, int nk) {
    gm.run(lds, PipeOperand{A, lda, va}, PipeOperand{B, ldb, vb}, nk);
}

// bf16: the tile of u' is staged in LDS as [token][feature] (512 bytes per token, 16-byte
// chunk c of token n in slot c ^ (n & 31)) and leaves as whole 512-byte row segments of H.
// fp32: each lane stores its 4 consecutive features directly.
template <typename T> struct MapStage { static constexpr bool kLds = false; static constexpr int kBytes = 0; };
template <> struct MapStage<bf16_t> { static constexpr bool kLds = true; static constexpr int kBytes = kTT * kFT * 2; };

// Q8 (bf16 only): the map is weight-only int8, codes packed like the bf16 map with one byte per
// element and one fp32 scale per row: the product runs on the codes (widened to bf16 in
// registers, exactly) and each row of it is multiplied by its scale before the intercept.
template <typename T, bool Q8 = false>
__global__ __launch_bounds__(MapCore<T>::G::kThr) void k_fill_map(MapArgs a) {
    using G = typename MapCore<T>::G;
    static_assert(!Q8 || std::is_same<T, bf16_t>::value, "int8 maps with bf16 prompt states");
    constexpr int kWaveRows = G::kThr / 64 / G::WGN;
    constexpr int kRedOff = MapStage<T>::kBytes;  // [kWaveRows][kTT] fp32 partial sums after the stage
    constexpr int kEpi = kRedOff + kWaveRows * kTT * 4;
    constexpr int kLdsBytes = G::LDS_BYTES > kEpi ? G::LDS_BYTES : kEpi;
    __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];
    int g, mt, tt;
    fill_tile(a.d / kFT, a.tok_tiles, g, mt, tt);
    const int64_t n0 = (int64_t)tt * kTT;
    G gm;
    if constexpr (Q8)
        gm.template run<false, false, false, true>(
            lds, PipeOperand{(const int8_t*)a.W[g] + (int64_t)mt * kFT * a.d, a.d, kFT},
            PipeOperand{(const T*)a.X + n0 * a.ldx, a.ldx, a.rows - n0}, a.d / G::BK);
    else
        fill_gemm(gm, lds, (const T*)a.W[g] + (int64_t)mt * kFT * a.d, a.d, kFT, (const T*)a.X + n0 * a.ldx, a.ldx,
                  a.rows - n0, a.d / G::BK);

    // the main loop ended on a barrier: LDS is free
    const int lane = threadIdx.x & 63;
    const int wm = (threadIdx.x >> 6) / G::WGN;   // wave row
    float* red = (float*)(lds + kRedOff);
    // bias and gamma of this lane's SM x 4 groups of 4 features, read once (16-byte loads) before any
    // staging write, so no LDS read waits behind the writes
    f32x4 bb[G::SM][4], gg[G::SM][4], sc[G::SM][4];
#pragma unroll
    for (int i = 0; i < G::SM; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int f = mt * kFT + G::row_of(i, 4 * q);
            bb[i][q] = *(const f32x4*)(a.bias[g] + f);
            gg[i][q] = *(const f32x4*)(a.gamma[g] + f);
            if constexpr (Q8) sc[i][q] = *(const f32x4*)(a.scale[g] + f);
        }
    T* H = (T*)a.H + g * a.h_slot;
#pragma unroll
    for (int j = 0; j < G::SN; ++j) {
        const int nl = G::col_of(j);
        const int64_t n = n0 + nl;
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < G::SM; ++i) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int ml = G::row_of(i, 4 * q);
                float h[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if constexpr (Q8) h[e] = gm.acc[i][j][4 * q + e] * sc[i][q][e] + bb[i][q][e];
                    else h[e] = gm.acc[i][j][4 * q + e] + bb[i][q][e];
                    ss += h[e] * h[e];
                }
                const f32x4 gq = gg[i][q];
                if constexpr (MapStage<T>::kLds) {
                    const int slot = ((ml >> 3) ^ (nl & 31)) << 4;
                    *(u32x2*)(lds + nl * (kFT * 2) + slot + (ml & 4) * 2) =
                        u32x2{pack_bf16x2(h[0] * gq[0], h[1] * gq[1]), pack_bf16x2(h[2] * gq[2], h[3] * gq[3])};
                } else {
                    if (n < a.rows)
                        store4<T>(H + n * a.d + (int64_t)mt * kFT + ml, h[0] * gq[0], h[1] * gq[1],
                                  h[2] * gq[2], h[3] * gq[3]);
                }
            }
        }
        ss += __shfl_xor(ss, 32);
        if (lane < 32) red[wm * kTT + nl] = ss;
    }
    __syncthreads();
    if constexpr (MapStage<T>::kLds) {
        // kThr / 32 tokens per pass; the 32 lanes of a half-wave write one token's 512 bytes
        constexpr int kTok = G::kThr / 32;
        const int c = threadIdx.x & 31;
#pragma unroll 4
        for (int p = 0; p < kTT / kTok; ++p) {
            const int nl = p * kTok + (threadIdx.x >> 5);
            const int64_t n = n0 + nl;
            const u32x4 v = *(const u32x4*)(lds + nl * (kFT * 2) + ((c ^ (nl & 31)) << 4));
            if (n < a.rows) *(u32x4*)(H + n * a.d + (int64_t)mt * kFT + c * 8) = v;
        }
    }
    {
        const int nl = threadIdx.x;
        const int64_t n = n0 + nl;
        if (nl < kTT && n < a.rows) {
            float ps = 0.f;
#pragma unroll
            for (int w = 0; w < kWaveRows; ++w) ps += red[w * kTT + nl];
            a.psum[g * a.ps_slot + n * a.n_ps + mt] = ps;
        }
    }
}

// The bf16 K/V product on 512-feature x 128-token tiles (PackedAGemm4), for widths whose K
// and V halves are whole 512-feature tiles: the same epilogue as k_fill_kv below (row scale,
// intercept, per-head key norm, RoPE, LDS-staged cache rows).  Wave w holds pairs of blocks
// (2p, 2p + 1), p = 0, 1, of the packed 64-row group ow = 2 (w % 2) + p of the 256-feature
// half w / 2: block 2p the low dims of the group's 32 RoPE pairs, block 2p + 1 their partners.
// A 128-wide head is one wave's two groups; a 64-wide head one group.
constexpr int kFT4 = 512, kTT4 = 128;
template <int DH, bool NORM, bool BIAS, bool KN>
__global__ __launch_bounds__(PackedAGemm4::kThr) void k_fill_kv4(KVArgs a) {
    using G = PackedAGemm4;
    constexpr int HALF = DH / 2;
    // LDS after the main loop: the staged rows of 64 tokens [token][feature] (1 KiB per token;
    // the tile is written in two halves), the tile's RoPE rows (DH floats per token, filled
    // during the main loop: the pipeline uses only the first 32 KiB), then 1/rms and the cache
    // row offset of every token of the tile
    constexpr int kHalfTok = kTT4 / 2;
    constexpr int kTab = kHalfTok * kFT4 * 2;
    constexpr int kTabRow = DH * 4;                        // bytes per token
    constexpr int kRinv = kTab + kTT4 * kTabRow;
    constexpr int kEpi = kRinv + kTT4 * 4 + kTT4 * 8;
    static_assert(G::LDS_BYTES <= kTab, "the RoPE rows must not overlap the pipeline stages");
    static_assert(kEpi <= 160 * 1024, "LDS");
    __shared__ __attribute__((aligned(16))) char lds[kEpi];
    const int n_feat = 2 * a.kvw / kFT4;
    const int per_layer = n_feat * a.tok_tiles;
    const int v = xcd_order((int)blockIdx.x, (int)gridDim.x);
    const int g = v / per_layer;
    int mt, tt;
    grouped_tile(v - g * per_layer, n_feat, a.tok_tiles, 4, mt, tt);
    const int64_t n0 = (int64_t)tt * kTT4;
    const bool is_k = (int64_t)mt * kFT4 < a.kvw;
    const int f0 = is_k ? mt * kFT4 : mt * kFT4 - a.kvw;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t nv = a.rows - n0 < kTT4 ? a.rows - n0 : kTT4;
    // RoPE rows of the tile's tokens straight into LDS (no registers, no wait here: the main
    // loop's first wait covers them).  16-byte chunk c of token n sits in slot c ^ (n % CPR); a
    // wave's load fills 1 KiB, TPB whole token rows; tokens past the end read as zero
    constexpr int CPR = DH / 4, TPB = 64 / CPR;
    if (is_k && a.rope) {
        const __amdgpu_buffer_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(a.rope + (a.pos0 + a.t0 + n0) * (int64_t)DH), (short)0, (int)(nv * kTabRow), 0x00020000);
        const int sl = lane % CPR;
#pragma unroll
        for (int u = 0; u < kTT4 / TPB / 4; ++u) {
            const int blk = w * (kTT4 / TPB / 4) + u;
            const int nl = blk * TPB + lane / CPR;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rr, (__attribute__((address_space(3))) void*)(lds + kTab + blk * 1024), 16,
                nl * kTabRow + ((sl ^ (nl % CPR)) << 4), 0, 0, 0);
        }
    }
    const bf16_t* Wsel = (const bf16_t*)(is_k ? a.Wk[g] : a.Wv[g]) + (int64_t)f0 * a.d;
    const bf16_t* Bsel = (const bf16_t*)(is_k ? a.in_k[g] : a.in_v[g]) + n0 * a.ld_in;
    G gm;
    gm.run(lds, PipeOperand{Wsel, a.d, kFT4}, PipeOperand{Bsel, a.ld_in, a.rows - n0}, a.d / G::BK);

    bf16_t* pool = (bf16_t*)(is_k ? a.kc[g] : a.vc[g]);
    const float* ps = NORM ? a.psum + g * a.ps_slot : nullptr;
    const float* bsel = BIAS ? (is_k ? a.bk[g] : a.bv[g]) + f0 : nullptr;
    const float inv_d = 1.0f / (float)a.d;
    auto rms_inv = [&](int64_t n) {
        if constexpr (!NORM) return 1.0f;
        float s = 0.f;
        if (a.n_ps % 4 == 0) {
            for (int p = 0; p < a.n_ps; p += 16) {
                f32x4 vv[4];
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    vv[u] = p + 4 * u < a.n_ps ? *(const f32x4*)(ps + n * a.n_ps + p + 4 * u) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    s += vv[u][0]; s += vv[u][1]; s += vv[u][2]; s += vv[u][3];
                }
            }
        } else {
            for (int p = 0; p < a.n_ps; ++p) s += ps[n * a.n_ps + p];
        }
        if (a.qb[g]) s += *a.qb[g];
        return 1.0f / sqrtf(s * inv_d + a.eps);
    };
    auto row_base = [&](int64_t t) -> int64_t {
        if (!a.paged) return t * a.stride_token;
        const int64_t lb = t / a.block_size;
        const int64_t phys = lb < a.n_table_blocks ? (int64_t)a.block_table[lb] : -1;
        if (phys < 0 || phys >= a.n_blocks) return -1;
        return phys * a.stride_block + (t % a.block_size) * a.stride_token;
    };
    float* rinv = (float*)(lds + kRinv);
    int64_t* rbase = (int64_t*)(lds + kRinv + kTT4 * 4);
    for (int nl = threadIdx.x; nl < kTT4; nl += G::kThr) {
        const bool ok = nl < nv;
        if constexpr (NORM) rinv[nl] = ok ? rms_inv(n0 + nl) : 0.f;
        rbase[nl] = ok ? row_base(a.t0 + n0 + nl) : -1;
    }
    __syncthreads();
    // [token][feature] for the 64 tokens of one half, 16-byte chunk c of token n in slot c ^ n
    auto stage = [&](int nh, int fl, const float (&o)[4]) {
        const int slot = ((fl >> 3) ^ nh) << 4;
        *(u32x2*)(lds + nh * (kFT4 * 2) + slot + (fl & 4) * 2) = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
    };
    const int half = w >> 1;                               // 256-feature half of the tile
    auto bias4 = [&](int fl) {
        if constexpr (BIAS) return *(const f32x4*)(bsel + fl);
        return f32x4{0.f, 0.f, 0.f, 0.f};
    };
    // lane's first RoPE pair of group p (within its 256-feature half) and the feature of pair qp
    auto qpair0 = [&](int p) { return (2 * (w & 1) + p) * 32 + 4 * (lane >> 5); };
    auto feat = [&](int qp) { return half * 256 + (qp / HALF) * DH + qp % HALF; };
    // per-head key norm weights of the lane's pairs (for the whole tile)
    f32x4 glo[2][4], ghi[2][4];
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int q = 0; q < 4; ++q) glo[p][q] = ghi[p][q] = f32x4{1.f, 1.f, 1.f, 1.f};
    if constexpr (KN) {
        if (is_k) {
#pragma unroll
            for (int p = 0; p < 2; ++p)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int qp = qpair0(p) + 8 * q;
                    glo[p][q] = *(const f32x4*)(a.kn[g] + qp % HALF);
                    ghi[p][q] = *(const f32x4*)(a.kn[g] + qp % HALF + HALF);
                }
        }
    }
    // whole 16-byte pieces of (token, head) rows: chunk c = features 8c .. 8c + 7 of the tile
    const int c = threadIdx.x & 63;
    const int head = (f0 + c * 8) / DH, dim = (f0 + c * 8) % DH;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int jj = 0; jj < G::SN / 2; ++jj) {
            const int j = h * (G::SN / 2) + jj;
            const int nh = jj * 32 + (lane & 31);          // token within the half
            const int nl = h * kHalfTok + nh;
            const float r = NORM ? rinv[nl] : 1.f;
            // the block pairs' values, scaled and with their intercepts
            float xlo[2][4][4], xhi[2][4][4];
#pragma unroll
            for (int p = 0; p < 2; ++p)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int fl = feat(qpair0(p) + 8 * q);
                    const f32x4 blo = bias4(fl), bhi = bias4(fl + HALF);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        xlo[p][q][e] = (gm.acc[2 * p][j][4 * q + e] + blo[e]) * r;
                        xhi[p][q][e] = (gm.acc[2 * p + 1][j][4 * q + e] + bhi[e]) * r;
                    }
                }
            if (!is_k) {
#pragma unroll
                for (int p = 0; p < 2; ++p)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int fl = feat(qpair0(p) + 8 * q);
                        stage(nh, fl, xlo[p][q]);
                        stage(nh, fl + HALF, xhi[p][q]);
                    }
                continue;
            }
            // keys: per-head norm (a 128-wide head: both groups of the wave; 64-wide: one
            // group), over the lane, the lane holding the token's other pairs (lane ^ 32)
            float kinv[2] = {1.f, 1.f};
            if constexpr (KN) {
                float ss[2] = {0.f, 0.f};
#pragma unroll
                for (int p = 0; p < 2; ++p)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
#pragma unroll
                        for (int e = 0; e < 4; ++e) ss[p] += xlo[p][q][e] * xlo[p][q][e] + xhi[p][q][e] * xhi[p][q][e];
                ss[0] += __shfl_xor(ss[0], 32);
                ss[1] += __shfl_xor(ss[1], 32);
                if constexpr (DH == 128) {
                    const float t = 1.0f / sqrtf((ss[0] + ss[1]) * (1.0f / (float)DH) + a.kn_eps);
                    kinv[0] = kinv[1] = t;
                } else {
                    kinv[0] = 1.0f / sqrtf(ss[0] * (1.0f / (float)DH) + a.kn_eps);
                    kinv[1] = 1.0f / sqrtf(ss[1] * (1.0f / (float)DH) + a.kn_eps);
                }
            }
#pragma unroll
            for (int p = 0; p < 2; ++p)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int qp = qpair0(p) + 8 * q;
                    const int fl = feat(qp);
                    // (cos, sin) of the lane's four pairs from the tile's RoPE rows; no table:
                    // the identity turn
                    f32x4 c01{1.f, 0.f, 1.f, 0.f}, c23{1.f, 0.f, 1.f, 0.f};
                    if (a.rope) {
                        const int c0 = (qp % HALF) / 2;
                        const char* row = lds + kTab + nl * kTabRow;
                        c01 = *(const f32x4*)(row + ((c0 ^ (nl % CPR)) << 4));
                        c23 = *(const f32x4*)(row + (((c0 + 1) ^ (nl % CPR)) << 4));
                    }
                    const float cs[4] = {c01[0], c01[2], c23[0], c23[2]};
                    const float sn[4] = {c01[1], c01[3], c23[1], c23[3]};
                    float lo[4], hi[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        float x = xlo[p][q][e], y = xhi[p][q][e];
                        if constexpr (KN) {
                            x *= kinv[p] * glo[p][q][e];
                            y *= kinv[p] * ghi[p][q][e];
                        }
                        lo[e] = x * cs[e] - y * sn[e];
                        hi[e] = y * cs[e] + x * sn[e];
                    }
                    stage(nh, fl, lo);
                    stage(nh, fl + HALF, hi);
                }
        }
        __syncthreads();
#pragma unroll 2
        for (int pz = 0; pz < kHalfTok / 4; ++pz) {
            const int nh = pz * 4 + w;
            const int64_t base = rbase[h * kHalfTok + nh];
            if (base < 0) continue;
            const u32x4 val = *(const u32x4*)(lds + nh * (kFT4 * 2) + ((c ^ nh) << 4));
            *(u32x4*)(pool + base + head * a.stride_head + dim) = val;
        }
        if (h == 0) __syncthreads();
    }
}

// NORM: the fill (rows scaled by 1/rms from the map's partial sums).  Otherwise the product
// of a translator (KV-Lingo page, section 3.1): no row scale, an intercept when BIAS.  HW
// (bf16): head-wise maps, block-diagonal by head, so a 256-feature tile reads only its own
// 256-column block of each source layer (d = nu * kvw; the other blocks are zero).  KN: keys
// are RMS-normalised per head with weights kn (KV-Lingo page, section 2) before the rotation.
template <typename T, int DH, bool NORM, bool BIAS, bool HW = false, bool KN = false>
__global__ __launch_bounds__(KVCore<T>::G::kThr) void k_fill_kv(KVArgs a) {
    using G = typename KVCore<T>::G;
    static_assert(!HW || (sizeof(T) == 2 && !NORM), "head-wise products are bf16 translators");
    static_assert(sizeof(T) == 2 || G::WTM % DH == 0, "fp32: a wave's feature extent must hold whole heads");
    static_assert(sizeof(T) == 4 || G::SM == 2, "bf16: the two blocks of a wave hold the RoPE partners");
    constexpr int HALF = DH / 2;
    constexpr int PAIR = HALF / 32;  // fp32: sub-tile distance between RoPE partners
    // staged tile, then 1/rms and the cache row offset of every token of the tile
    // (KN: then the per-wave, per-token partial key sums of squares)
    constexpr int kEpi = sizeof(T) == 2 ? kTT * kFT * 2 + kTT * 4 + kTT * 8 + (KN ? 4 * kTT * 4 : 0) : 0;
    __shared__ __attribute__((aligned(16))) char lds[G::LDS_BYTES > kEpi ? G::LDS_BYTES : kEpi];
    int g, mt, tt;
    fill_tile(2 * a.kvw / kFT, a.tok_tiles, g, mt, tt);
    const int64_t n0 = (int64_t)tt * kTT;
    const bool is_k = (int64_t)mt * kFT < a.kvw;
    const int f0 = is_k ? mt * kFT : mt * kFT - a.kvw;
    const T* Wsel = (const T*)(is_k ? a.Wk[g] : a.Wv[g]) + (int64_t)f0 * a.d;
    const T* Bsel = (const T*)(is_k ? a.in_k[g] : a.in_v[g]) + n0 * a.ld_in;
    G gm;
    if constexpr (HW) {
        // segments of 4 k-steps (the tile's 256 source columns), one per source layer
        gm.template run<false, true>(lds, PipeOperand{Wsel + (int64_t)(f0 / G::BK) * (G::kStepBytes / 2), a.d, kFT},
                                     PipeOperand{Bsel + f0, a.ld_in, a.rows - n0}, 4 * (a.d / a.kvw), 0,
                                     a.kvw / G::BK);
    } else {
        fill_gemm(gm, lds, Wsel, a.d, kFT, Bsel, a.ld_in, a.rows - n0, a.d / G::BK);
    }

    T* pool = (T*)(is_k ? a.kc[g] : a.vc[g]);
    const float* ps = NORM ? a.psum + g * a.ps_slot : nullptr;
    const float* bsel = BIAS ? (is_k ? a.bk[g] : a.bv[g]) + f0 : nullptr;
    const float inv_d = 1.0f / (float)a.d;
    // 1 / rms of token n from its per-feature-tile partial sums (fixed order)
    auto rms_inv = [&](int64_t n) {
        if constexpr (!NORM) return 1.0f;
        float s = 0.f;
        if (a.n_ps % 4 == 0) {
            // four independent loads per pass, added in index order
            for (int p = 0; p < a.n_ps; p += 16) {
                f32x4 v[4];
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    v[u] = p + 4 * u < a.n_ps ? *(const f32x4*)(ps + n * a.n_ps + p + 4 * u) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    s += v[u][0]; s += v[u][1]; s += v[u][2]; s += v[u][3];
                }
            }
        } else {
            for (int p = 0; p < a.n_ps; ++p) s += ps[n * a.n_ps + p];
        }
        if (a.qb[g]) s += *a.qb[g];   // composed maps: the constant term of the sum of squares
        return 1.0f / sqrtf(s * inv_d + a.eps);
    };
    // element offset of token t's row in the pool, or -1 if it has no slot
    auto row_base = [&](int64_t t) -> int64_t {
        if (!a.paged) return t * a.stride_token;
        const int64_t lb = t / a.block_size;
        const int64_t phys = lb < a.n_table_blocks ? (int64_t)a.block_table[lb] : -1;
        if (phys < 0 || phys >= a.n_blocks) return -1;
        return phys * a.stride_block + (t % a.block_size) * a.stride_token;
    };
    // final values: scaled by r = 1/rms of their token; keys rotated by their position
    if constexpr (sizeof(T) == 2) {
        // 1/rms and the cache row offset of the tile's tokens, once per token, after the
        // staging area (read from LDS below, so no global load follows a cache store)
        float* rinv = (float*)(lds + kTT * kFT * 2);
        int64_t* rbase = (int64_t*)(lds + kTT * kFT * 2 + kTT * 4);
        for (int nl = threadIdx.x; nl < kTT; nl += G::kThr) {
            const bool ok = n0 + nl < a.rows;
            if constexpr (NORM) rinv[nl] = ok ? rms_inv(n0 + nl) : 0.f;
            rbase[nl] = ok ? row_base(a.t0 + n0 + nl) : -1;
        }
        __syncthreads();
        // bf16: stage the 256 tokens x 256 features tile in LDS ([token][feature], 16-byte
        // chunk c of token n in slot c ^ (n & 31)), then write whole (token, head) rows
        auto stage = [&](int nl, int fl, const float (&o)[4]) {
            const int slot = ((fl >> 3) ^ (nl & 31)) << 4;
            *(u32x2*)(lds + nl * (kFT * 2) + slot + (fl & 4) * 2) =
                u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
        };
        // packed rows: block 0 of wave wm holds low dims of pairs 32 wm + (row % 32), block 1
        // their partners (dims + HALF), in the same registers
        const int wm = threadIdx.x >> 6;
        const int qp0 = wm * 32 + 4 * ((threadIdx.x & 63) >> 5);
        // intercepts of 4 features from fl (read where used: cache hits, no registers held)
        auto bias4 = [&](int fl) {
            if constexpr (BIAS) return *(const f32x4*)(bsel + fl);
            return f32x4{0.f, 0.f, 0.f, 0.f};
        };
        // per-head key norm: a wave's 32 pairs are half of a 128-wide head (the other half in
        // wave wm ^ 1) or all of a 64-wide one; each token's sum of squares over the lane's 32
        // values, the lane holding the token's other pairs (lane ^ 32) and, for 128, the partner
        // wave (through LDS) gives 1/rms of the head
        float* knred = (float*)(lds + kTT * kFT * 2 + kTT * 4 + kTT * 8);
        if constexpr (KN) {
            if (is_k) {
#pragma unroll
                for (int j = 0; j < G::SN; ++j) {
                    const int nl = G::col_of(j);
                    const float r = NORM ? rinv[nl] : 1.f;
                    float ss = 0.f;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int qp = qp0 + 8 * q;
                        const int fl = (qp / HALF) * DH + qp % HALF;
                        const f32x4 blo = bias4(fl), bhi = bias4(fl + HALF);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float x = (gm.acc[0][j][4 * q + e] + blo[e]) * r;
                            const float y = (gm.acc[1][j][4 * q + e] + bhi[e]) * r;
                            ss += x * x + y * y;
                        }
                    }
                    ss += __shfl_xor(ss, 32);
                    if ((threadIdx.x & 63) < 32) knred[wm * kTT + nl] = ss;
                }
                __syncthreads();
            }
        }
#pragma unroll
        for (int j = 0; j < G::SN; ++j) {
            const int nl = G::col_of(j);
            const int64_t n = n0 + nl;
            const float r = NORM ? rinv[nl] : 1.f;
            if (!is_k) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int qp = qp0 + 8 * q;
                    const int fl = (qp / HALF) * DH + qp % HALF;
                    const f32x4 blo = bias4(fl), bhi = bias4(fl + HALF);
                    float lo[4], hi[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        lo[e] = (gm.acc[0][j][4 * q + e] + blo[e]) * r;
                        hi[e] = (gm.acc[1][j][4 * q + e] + bhi[e]) * r;
                    }
                    stage(nl, fl, lo);
                    stage(nl, fl + HALF, hi);
                }
            } else {
                // (cos, sin) of the lane's 4 x 4 low dims, loaded together ahead of their uses;
                // no table (translators of rotated keys): the identity turn
                f32x4 c01[4], c23[4];
                if (a.rope) {
                    const float* cs_row = a.rope + (a.pos0 + a.t0 + (n < a.rows ? n : 0)) * (int64_t)DH;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int dlo = (qp0 + 8 * q) % HALF;
                        c01[q] = *(const f32x4*)(cs_row + 2 * dlo);
                        c23[q] = *(const f32x4*)(cs_row + 2 * dlo + 4);
                    }
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q) c01[q] = c23[q] = f32x4{1.f, 0.f, 1.f, 0.f};
                }
                __builtin_amdgcn_sched_barrier(0);
                float kinv = 1.f;
                if constexpr (KN) {
                    float ssh = knred[wm * kTT + nl];
                    if constexpr (DH == 128) ssh += knred[(wm ^ 1) * kTT + nl];
                    kinv = 1.0f / sqrtf(ssh * (1.0f / (float)DH) + a.kn_eps);
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int qp = qp0 + 8 * q;
                    const int fl = (qp / HALF) * DH + qp % HALF;
                    const float cs[4] = {c01[q][0], c01[q][2], c23[q][0], c23[q][2]};
                    const float sn[4] = {c01[q][1], c01[q][3], c23[q][1], c23[q][3]};
                    const f32x4 blo = bias4(fl), bhi = bias4(fl + HALF);
                    f32x4 glo{1.f, 1.f, 1.f, 1.f}, ghi{1.f, 1.f, 1.f, 1.f};
                    if constexpr (KN) {
                        glo = *(const f32x4*)(a.kn[g] + qp % HALF);
                        ghi = *(const f32x4*)(a.kn[g] + qp % HALF + HALF);
                    }
                    float lo[4], hi[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        float x = (gm.acc[0][j][4 * q + e] + blo[e]) * r;
                        float y = (gm.acc[1][j][4 * q + e] + bhi[e]) * r;
                        if constexpr (KN) {
                            x *= kinv * glo[e];
                            y *= kinv * ghi[e];
                        }
                        lo[e] = x * cs[e] - y * sn[e];
                        hi[e] = y * cs[e] + x * sn[e];
                    }
                    stage(nl, fl, lo);
                    stage(nl, fl + HALF, hi);
                }
            }
        }
        __syncthreads();
        constexpr int kTok = G::kThr / 32;
        const int c = threadIdx.x & 31;            // 16-byte chunk: features 8c .. 8c+7
        const int head = (f0 + c * 8) / DH, dim = (f0 + c * 8) % DH;
#pragma unroll 2
        for (int p = 0; p < kTT / kTok; ++p) {
            const int nl = p * kTok + (threadIdx.x >> 5);
            const int64_t base = rbase[nl];     // -1: past the rows, or no cache slot
            if (base < 0) continue;
            const u32x4 v = *(const u32x4*)(lds + nl * (kFT * 2) + ((c ^ (nl & 31)) << 4));
            *(u32x4*)(pool + base + head * a.stride_head + dim) = v;
        }
    } else {
        // fp32: each lane stores its 4 consecutive features directly
#pragma unroll
        for (int j = 0; j < G::SN; ++j) {
            const int64_t n = n0 + G::col_of(j);
            if (n >= a.rows) continue;
            const int64_t t = a.t0 + n;
            const int64_t base = row_base(t);
            if (base < 0) continue;
            const float r = rms_inv(n);
            // HALF (cos, sin) pairs; no table: the identity turn
            const float* cs_row = a.rope ? a.rope + (a.pos0 + t) * (int64_t)DH : nullptr;
            // per-head key norm: sub-tiles i of one head (DH / 32 of them, inside the wave's
            // rows) and the token's other rows in lane ^ 32
            float kinv[G::SM];
#pragma unroll
            for (int i = 0; i < G::SM; ++i) kinv[i] = 1.f;
            if constexpr (KN) {
                if (is_k) {
                    constexpr int kSub = DH / 32;
#pragma unroll
                    for (int h0 = 0; h0 < G::SM; h0 += kSub) {
                        float ss = 0.f;
#pragma unroll
                        for (int i = h0; i < h0 + kSub; ++i)
#pragma unroll
                            for (int q = 0; q < 4; ++q)
#pragma unroll
                                for (int e = 0; e < 4; ++e) {
                                    float x = gm.acc[i][j][4 * q + e] * r;
                                    if constexpr (BIAS) x += bsel[G::row_of(i, 4 * q) + e];
                                    ss += x * x;
                                }
                        ss += __shfl_xor(ss, 32);
                        const float inv = 1.0f / sqrtf(ss * (1.0f / (float)DH) + a.kn_eps);
#pragma unroll
                        for (int i = h0; i < h0 + kSub; ++i) kinv[i] = inv;
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < G::SM; ++i) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int f = f0 + G::row_of(i, 4 * q);
                    const int head = f / DH;
                    const int dim = f % DH;
                    T* dst = pool + base + head * a.stride_head + dim;
                    const int fb = f - f0;  // intercept index of this lane's first feature
                    auto add_b = [&](float v, int idx) {
                        if constexpr (BIAS) return v + bsel[idx];
                        return v;
                    };
                    if (!is_k) {
                        store4<T>(dst, add_b(gm.acc[i][j][4 * q] * r, fb), add_b(gm.acc[i][j][4 * q + 1] * r, fb + 1),
                                  add_b(gm.acc[i][j][4 * q + 2] * r, fb + 2), add_b(gm.acc[i][j][4 * q + 3] * r, fb + 3));
                    } else if ((i * 32) % DH < HALF) {
                        // this sub-tile holds dims [dim, dim+4) < HALF; partner sub-tile i+PAIR
                        // holds dims + HALF of the same head in the same registers
                        const f32x4 c01 = cs_row ? *(const f32x4*)(cs_row + 2 * dim) : f32x4{1.f, 0.f, 1.f, 0.f};
                        const f32x4 c23 = cs_row ? *(const f32x4*)(cs_row + 2 * dim + 4) : f32x4{1.f, 0.f, 1.f, 0.f};
                        const float cs[4] = {c01[0], c01[2], c23[0], c23[2]};
                        const float sn[4] = {c01[1], c01[3], c23[1], c23[3]};
                        float lo[4], hi[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            float x0 = add_b(gm.acc[i][j][4 * q + e] * r, fb + e);
                            float x1 = add_b(gm.acc[(i + PAIR) % G::SM][j][4 * q + e] * r, fb + HALF + e);
                            if constexpr (KN) {
                                x0 *= kinv[i] * a.kn[g][dim + e];
                                x1 *= kinv[(i + PAIR) % G::SM] * a.kn[g][dim + HALF + e];
                            }
                            lo[e] = x0 * cs[e] - x1 * sn[e];
                            hi[e] = x1 * cs[e] + x0 * sn[e];
                        }
                        store4<T>(dst, lo[0], lo[1], lo[2], lo[3]);
                        store4<T>(dst + HALF, hi[0], hi[1], hi[2], hi[3]);
                    }
                }
            }
        }
    }
}


// ---- the composed fill: the maps folded into the layers' projections -----------------------
// With W' = W_k,v diag(gamma) W (composed once per map, rf_fill_compose), a token's keys and
// values are (x W'^T + c) r, where c = W_k,v diag(gamma) b and r = 1/rms(h) needs only the sum
// of squares of h = x W^T + b:
//     sum_o h_o^2 = x G x^T + x (2 W^T b) + |b|^2,   G = W^T W,
// a quadratic form read with the strictly upper-triangular T (T_ij = 2 G_ij for j > i) and
// G's diagonal kept in fp32: x G x^T = sum_i x_i ((T x)_i + G_ii x_i).  k_fill_norm forms
// (T x)_i over 256-feature tiles, reading only columns j >= the tile's first feature (T is zero
// to their left), and leaves the tile's partial  sum_i x_i ((T x)_i + G_ii x_i + 2 (W^T b)_i)
// per token; the K/V launch reads X itself.
struct NormArgs {
    const void* X;
    int64_t ldx;
    int64_t rows;
    int32_t d;
    int32_t n_ps;            // partial sums per token = d / kFT
    int32_t tok_tiles;
    int32_t n_layers;
    float* psum;             // [rows][n_ps] per layer slot
    int64_t ps_slot;
    const void* T[kMaxGroup];   // packed [d][d] (upper block triangle read)
    const float* q[kMaxGroup];  // [2d + 1]: 2 W^T b, diag(W^T W), then |b|^2
};

__global__ __launch_bounds__(PackedAGemm::kThr) void k_fill_norm(NormArgs a) {
    using G = PackedAGemm;
    // epilogue: the tile's x values [token][feature] (bf16, 16-byte chunk c of token n in slot
    // c ^ (n & 31)), then the [wave][token] fp32 partials
    constexpr int kX = kTT * kFT * 2, kRed = 4 * kTT * 4;
    constexpr int kEpi = kX + kRed;
    __shared__ __attribute__((aligned(16))) char lds[G::LDS_BYTES > kEpi ? G::LDS_BYTES : kEpi];
    const int n_feat = a.d / kFT;
    // the K range shrinks with the feature tile: every XCD takes a block of (layer, token tile)
    // columns with all their feature tiles, longest first, 4 feature x 8 token tiles at a time
    int mt, col;
    balanced_tile(xcd_order((int)blockIdx.x, (int)gridDim.x), n_feat, a.n_layers * a.tok_tiles, mt, col);
    const int g = col / a.tok_tiles, tt = col - g * a.tok_tiles;
    const int64_t n0 = (int64_t)tt * kTT;
    const int kb = mt * (kFT / G::BK);   // first k-step: column 256 mt
    const bf16_t* X = (const bf16_t*)a.X;
    G gm;
    // the K loop from the last column down: the row tiles of one token tile that run together
    // then read the same prompt-state columns at the same time (they all end at column d), and
    // the tile's own x block, read last, is still in the L2 for the epilogue
    gm.template run<false, false, true>(
        lds, PipeOperand{(const bf16_t*)a.T[g] + (int64_t)mt * kFT * a.d + (int64_t)kb * (G::kStepBytes / 2), a.d, kFT},
        PipeOperand{X + n0 * a.ldx + (int64_t)mt * kFT, a.ldx, a.rows - n0}, a.d / G::BK - kb);

    // the main loop ended on a barrier: LDS is free.  The tile's x values come back as whole
    // 512-byte row segments (a half-wave per token; rows past the end read as zero through the
    // buffer's range) and are read per lane from LDS in the accumulators' layout.  Sixteen loads
    // per thread are issued before the first LDS write: a load-then-write loop waits one memory
    // round trip per row pass, which cost more than the rest of the epilogue
    const int lane = threadIdx.x & 63, wm = threadIdx.x >> 6;
    {
        const int c = threadIdx.x & 31;
        const int64_t nv = a.rows - n0 < kTT ? a.rows - n0 : kTT;
        const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<bf16_t*>(X + n0 * a.ldx), (short)0, (int)(nv * a.ldx * 2), 0x00020000);
        constexpr int kInFlight = 16;
#pragma unroll
        for (int p0 = 0; p0 < kTT / 8; p0 += kInFlight) {
            u32x4 v[kInFlight];
#pragma unroll
            for (int u = 0; u < kInFlight; ++u) {
                const int nl = (p0 + u) * 8 + (threadIdx.x >> 5);
                v[u] = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)((nl * a.ldx + mt * kFT + c * 8) * 2), 0, 0);
            }
#pragma unroll
            for (int u = 0; u < kInFlight; ++u) {
                const int nl = (p0 + u) * 8 + (threadIdx.x >> 5);
                *(u32x4*)(lds + nl * (kFT * 2) + ((c ^ (nl & 31)) << 4)) = v[u];
            }
        }
    }
    __syncthreads();
    float* red = (float*)(lds + kX);
    const float* qv = a.q[g];
    f32x4 gq[G::SM][4], gd[G::SM][4];
#pragma unroll
    for (int i = 0; i < G::SM; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            gq[i][q] = *(const f32x4*)(qv + mt * kFT + G::row_of(i, 4 * q));
            gd[i][q] = *(const f32x4*)(qv + a.d + mt * kFT + G::row_of(i, 4 * q));
        }
#pragma unroll
    for (int j = 0; j < G::SN; ++j) {
        const int nl = G::col_of(j);
        const int64_t n = n0 + nl;
        // this lane's 32 features of the token's own row
        u32x2 xv[G::SM][4];
#pragma unroll
        for (int i = 0; i < G::SM; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int ml = G::row_of(i, 4 * q);
                xv[i][q] = *(const u32x2*)(lds + nl * (kFT * 2) + (((ml >> 3) ^ (nl & 31)) << 4) + (ml & 4) * 2);
            }
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < G::SM; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float x0 = __builtin_bit_cast(float, xv[i][q][0] << 16);
                const float x1 = __builtin_bit_cast(float, xv[i][q][0] & 0xffff0000u);
                const float x2 = __builtin_bit_cast(float, xv[i][q][1] << 16);
                const float x3 = __builtin_bit_cast(float, xv[i][q][1] & 0xffff0000u);
                ss += x0 * (gm.acc[i][j][4 * q] + gq[i][q][0] + gd[i][q][0] * x0);
                ss += x1 * (gm.acc[i][j][4 * q + 1] + gq[i][q][1] + gd[i][q][1] * x1);
                ss += x2 * (gm.acc[i][j][4 * q + 2] + gq[i][q][2] + gd[i][q][2] * x2);
                ss += x3 * (gm.acc[i][j][4 * q + 3] + gq[i][q][3] + gd[i][q][3] * x3);
            }
        if (n >= a.rows) ss = 0.f;
        ss += __shfl_xor(ss, 32);
        if (lane < 32) red[wm * kTT + nl] = ss;
        __builtin_amdgcn_sched_barrier(0);   // one token column at a time (register pressure)
    }
    __syncthreads();
    const int nl = threadIdx.x;
    const int64_t n = n0 + nl;
    if (nl < kTT && n < a.rows) {
        const float ps = ((red[nl] + red[kTT + nl]) + red[2 * kTT + nl]) + red[3 * kTT + nl];
        a.psum[g * a.ps_slot + n * a.n_ps + mt] = ps;
    }
}

__global__ void k_rope_table(double base, int32_t dh, int64_t p0, int64_t n_pos, float* out) {
    const int64_t half = dh / 2;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= n_pos * half) return;
    const int64_t p = idx / half;
    const int64_t i = idx % half;
    const double theta = pow(base, -2.0 * (double)i / (double)dh);
    const double phi = (double)(p0 + p) * theta;   // row p holds position p0 + p
    out[2 * idx] = (float)cos(phi);
    out[2 * idx + 1] = (float)sin(phi);
}


// 8 consecutive k of one source row as 8 bf16 (fp32 sources rounded to nearest even).
__device__ inline u32x4 load8_bf16(const bf16_t* p) { return *(const u32x4*)p; }
__device__ inline u32x4 load8_bf16(const float* p) {
    const f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
    return u32x4{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3])};
}

// One 16-byte chunk (8 consecutive k of one row) per thread, in packed order: writes are
// contiguous, reads are pieces of source rows.
template <typename S>
__global__ void k_pack_weights(const S* __restrict__ src, int64_t ld, int64_t cols, int32_t hd,
                               int64_t n_chunks, bf16_t* __restrict__ dst) {
    const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= n_chunks) return;
    const int64_t e = c * 8;
    const int64_t tile_elems = 256 * cols;
    const int64_t tile = e / tile_elems;
    const int64_t rem = e - tile * tile_elems;
    const int64_t kt = rem >> 14;                   // 16384 elements per k-step
    const int r2 = (int)(rem & 16383);
    const int w = r2 >> 12, kk = (r2 >> 10) & 3, i = (r2 >> 9) & 1, lane = (r2 >> 3) & 63;
    const int p = (w << 6) + (i << 5) + (lane & 31);
    const int64_t row = tile * 256 + packed_source_row(p, hd);
    const int64_t k = kt * 64 + kk * 16 + (lane >> 5) * 8;
    *(u32x4*)(dst + e) = load8_bf16(src + row * ld + k);
}

// Row-wise symmetric int8 codes of an fp32 map: one work-group per row; the row's absolute
// maximum by a work-group reduction, then each thread codes chunks of 8 consecutive columns
// and writes them as 8 bytes in packed order.  The code is rint(w / s) in fp32 (IEEE
// division, ties to even), clamped to [-127, 127].
__global__ __launch_bounds__(256) void k_quantize_map(const float* __restrict__ W, int64_t ld, int64_t cols,
                                                      int8_t* __restrict__ q, float* __restrict__ scale) {
    __shared__ float red[4];
    const int64_t row = blockIdx.x;
    const float* src = W + row * ld;
    float m = 0.f;
    for (int64_t c = threadIdx.x * 4; c < cols; c += 256 * 4) {
        const f32x4 v = *(const f32x4*)(src + c);
        m = fmaxf(m, fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    const float amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float s = amax / 127.0f;
    if (threadIdx.x == 0) scale[row] = s;
    const int64_t base = (row >> 8) * 256 * cols + packed_row_part((int)(row & 255));
    for (int64_t c = threadIdx.x * 8; c < cols; c += 256 * 8) {
        const f32x4 a = *(const f32x4*)(src + c), b = *(const f32x4*)(src + c + 4);
        const float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
        uint32_t wd[2] = {0u, 0u};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float r = s > 0.f ? fminf(fmaxf(rintf(x[e] / s), -127.f), 127.f) : 0.f;
            wd[e >> 2] |= ((uint32_t)(int)r & 0xffu) << (8 * (e & 3));
        }
        *(u32x2*)(q + base + packed_col_part((int)c)) = u32x2{wd[0], wd[1]};
    }
}

// Bytes at the end of a fill's workspace that hold the RoPE table of a call's tokens when the
// caller passes none.
static size_t rope_ws_bytes(int32_t head_dim, int64_t n_tokens) {
    return round_up((size_t)n_tokens * head_dim * sizeof(float), 256);
}

static size_t slot_bytes(const rf_fill_weights* w, int64_t rows) {
    const size_t hb = round_up((size_t)rows * w->d * elem_bytes(w->dtype), 256);
    const size_t pb = round_up((size_t)rows * (w->d / kFT) * sizeof(float), 256);
    return hb + pb;
}

// The K/V launch of a group of layers: the 512-feature x 128-token tile kernel for the bf16
// fills when the K and V halves are whole 512-feature tiles, else the 256 x 256 one.  (The
// translators, whose contraction is half as long, measured 2.6 % slower on the 512 x 128 tiles:
// 4.43 against 4.32 ms for 36 target layers of 16384 tokens.)
template <typename T, int DH, bool NORM, bool BIAS, bool KN>
static void launch_kv(KVArgs ka, int64_t rows, int gsz, hipStream_t stream) {
    if constexpr (sizeof(T) == 2 && NORM) {
        if (ka.kvw % kFT4 == 0) {
            ka.tok_tiles = (int32_t)ceil_div(rows, (int64_t)kTT4);
            hipLaunchKernelGGL((k_fill_kv4<DH, NORM, BIAS, KN>), dim3((unsigned)((2 * ka.kvw / kFT4) * ka.tok_tiles * gsz)),
                               dim3(PackedAGemm4::kThr), 0, stream, ka);
            return;
        }
    }
    ka.tok_tiles = (int32_t)ceil_div(rows, (int64_t)kTT);
    hipLaunchKernelGGL((k_fill_kv<T, DH, NORM, BIAS, false, KN>), dim3((unsigned)((2 * ka.kvw / kFT) * ka.tok_tiles * gsz)),
                       dim3(KVCore<T>::G::kThr), 0, stream, ka);
}

template <typename T>
static rf_status launch_fill(const rf_fill_weights* w, int32_t n_layers, const void* X, int64_t ldx,
                             int64_t t0, int64_t t1, int64_t pos0, const rf_cache_desc* cache,
                             const rf_cache_layout_t& L, void* const* kc, void* const* vc,
                             const int32_t* table, int64_t n_table, const float* rope, void* ws,
                             size_t ws_bytes, hipStream_t stream) {
    const int64_t rows = t1 - t0;
    const size_t slot = slot_bytes(w, rows);
    const int group = (int)std::min<size_t>({(size_t)n_layers, (size_t)kMaxGroup, ws_bytes / slot});
    const size_t hb = round_up((size_t)rows * w->d * sizeof(T), 256);
    char* wsc = (char*)ws;
    const int64_t h_slot = (int64_t)(slot / sizeof(T));
    const int64_t ps_slot = (int64_t)(slot / sizeof(float));
    const int tok_tiles = (int)ceil_div(rows, kTT);
    for (int l0 = 0; l0 < n_layers; l0 += group) {
        const int gsz = std::min(group, n_layers - l0);
        MapArgs ma{};
        ma.X = X; ma.ldx = ldx; ma.rows = rows; ma.d = w->d; ma.n_ps = w->d / kFT;
        ma.H = wsc; ma.h_slot = h_slot; ma.psum = (float*)(wsc + hb); ma.ps_slot = ps_slot;
        KVArgs ka{};
        ka.psum = (const float*)(wsc + hb); ka.ps_slot = ps_slot; ka.ld_in = w->d;
        ka.n_ps = w->d / kFT; ka.d = w->d; ka.kvw = w->n_kv_heads * w->head_dim; ka.eps = w->rms_eps;
        ka.rows = rows; ka.t0 = t0; ka.pos0 = pos0; ka.rope = rope;
        ka.paged = cache->layout == RF_LAYOUT_PAGED; ka.block_size = cache->block_size;
        ka.stride_block = L.stride_block; ka.stride_head = L.stride_head; ka.stride_token = L.stride_token;
        ka.n_blocks = L.n_blocks; ka.block_table = table; ka.n_table_blocks = n_table;
        ka.kn_eps = w->k_norm_eps;
        for (int g = 0; g < gsz; ++g) {
            ma.W[g] = w->W_map[l0 + g]; ma.bias[g] = w->b_map[l0 + g]; ma.gamma[g] = w->gamma[l0 + g];
            ma.scale[g] = w->map_scale ? w->map_scale[l0 + g] : nullptr;
            ka.kn[g] = w->k_norm ? w->k_norm[l0 + g] : nullptr;
            ka.Wk[g] = w->W_k[l0 + g]; ka.Wv[g] = w->W_v[l0 + g];
            ka.in_k[g] = ka.in_v[g] = (const T*)wsc + g * h_slot;
            ka.kc[g] = kc[l0 + g]; ka.vc[g] = vc[l0 + g];
        }
        ma.tok_tiles = tok_tiles;
        ka.tok_tiles = tok_tiles;
        bool launched = false;
        if constexpr (std::is_same<T, bf16_t>::value) {
            if (w->map_scale) {
                hipLaunchKernelGGL((k_fill_map<T, true>), dim3((w->d / kFT) * tok_tiles * gsz), dim3(MapCore<T>::G::kThr),
                                   0, stream, ma);
                launched = true;
            }
        }
        if (!launched)
            hipLaunchKernelGGL(k_fill_map<T>, dim3((w->d / kFT) * tok_tiles * gsz), dim3(MapCore<T>::G::kThr), 0, stream, ma);
        rf_status st = check_launch("rf_fill: map kernel");
        if (st != RF_OK) return st;
        if (w->k_norm) {
            if (w->head_dim == 128) launch_kv<T, 128, true, false, true>(ka, rows, gsz, stream);
            else launch_kv<T, 64, true, false, true>(ka, rows, gsz, stream);
        } else {
            if (w->head_dim == 128) launch_kv<T, 128, true, false, false>(ka, rows, gsz, stream);
            else launch_kv<T, 64, true, false, false>(ka, rows, gsz, stream);
        }
        st = check_launch("rf_fill: kv kernel");
        if (st != RF_OK) return st;
    }
    return RF_OK;
}


static size_t composed_slot_bytes(const rf_fill_composed_weights* w, int64_t rows) {
    return round_up((size_t)rows * (w->d / kFT) * sizeof(float), 256);
}

// Per group of layers: the quadratic-form launch, then the K/V launch reading the prompt
// states directly (the composed maps make the predicted inputs unnecessary).
static rf_status launch_fill_composed(const rf_fill_composed_weights* w, int32_t n_layers, const void* X, int64_t ldx,
                                      int64_t t0, int64_t t1, int64_t pos0, const rf_cache_desc* cache,
                                      const rf_cache_layout_t& L, void* const* kc, void* const* vc,
                                      const int32_t* table, int64_t n_table, const float* rope, void* ws,
                                      size_t ws_bytes, hipStream_t stream) {
    const int64_t rows = t1 - t0;
    const size_t slot = composed_slot_bytes(w, rows);
    const int group = (int)std::min<size_t>({(size_t)n_layers, (size_t)kMaxGroup, ws_bytes / slot});
    const int64_t ps_slot = (int64_t)(slot / sizeof(float));
    const int tok_tiles = (int)ceil_div(rows, kTT);
    const int kvw = w->n_kv_heads * w->head_dim;
    for (int l0 = 0; l0 < n_layers; l0 += group) {
        const int gsz = std::min(group, n_layers - l0);
        NormArgs na{};
        na.X = X; na.ldx = ldx; na.rows = rows; na.d = w->d; na.n_ps = w->d / kFT; na.tok_tiles = tok_tiles;
        na.n_layers = gsz; na.psum = (float*)ws; na.ps_slot = ps_slot;
        KVArgs ka{};
        ka.psum = (const float*)ws; ka.ps_slot = ps_slot; ka.ld_in = ldx;
        ka.n_ps = w->d / kFT; ka.d = w->d; ka.kvw = kvw; ka.eps = w->rms_eps;
        ka.rows = rows; ka.t0 = t0; ka.pos0 = pos0; ka.rope = rope;
        ka.paged = cache->layout == RF_LAYOUT_PAGED; ka.block_size = cache->block_size;
        ka.stride_block = L.stride_block; ka.stride_head = L.stride_head; ka.stride_token = L.stride_token;
        ka.n_blocks = L.n_blocks; ka.block_table = table; ka.n_table_blocks = n_table;
        ka.kn_eps = w->k_norm_eps;
        for (int g = 0; g < gsz; ++g) {
            na.T[g] = w->T[l0 + g]; na.q[g] = w->q[l0 + g];
            ka.qb[g] = w->q[l0 + g] + 2 * w->d;
            ka.kn[g] = w->k_norm ? w->k_norm[l0 + g] : nullptr;
            ka.Wk[g] = w->M_k[l0 + g]; ka.Wv[g] = w->M_v[l0 + g];
            ka.bk[g] = w->c_k[l0 + g]; ka.bv[g] = w->c_v[l0 + g];
            ka.in_k[g] = ka.in_v[g] = X;
            ka.kc[g] = kc[l0 + g]; ka.vc[g] = vc[l0 + g];
        }
        ka.tok_tiles = tok_tiles;
        hipLaunchKernelGGL(k_fill_norm, dim3((w->d / kFT) * tok_tiles * gsz), dim3(PackedAGemm::kThr), 0, stream, na);
        rf_status st = check_launch("rf_fill_composed: quadratic-form kernel");
        if (st != RF_OK) return st;
        if (w->k_norm) {
            if (w->head_dim == 128) launch_kv<bf16_t, 128, true, true, true>(ka, rows, gsz, stream);
            else launch_kv<bf16_t, 64, true, true, true>(ka, rows, gsz, stream);
        } else {
            if (w->head_dim == 128) launch_kv<bf16_t, 128, true, true, false>(ka, rows, gsz, stream);
            else launch_kv<bf16_t, 64, true, true, false>(ka, rows, gsz, stream);
        }
        st = check_launch("rf_fill_composed: kv kernel");
        if (st != RF_OK) return st;
    }
    return RF_OK;
}

template <typename T, int DH, bool BIAS, bool KN>
static void launch_translate_group(const KVArgs& ka, int gsz, bool headwise, hipStream_t stream) {
    const dim3 grid((2 * ka.kvw / kFT) * ka.tok_tiles * gsz);
    if constexpr (sizeof(T) == 2) {
        if (headwise) {
            hipLaunchKernelGGL((k_fill_kv<T, DH, false, BIAS, true, KN>), grid, dim3(KVCore<T>::G::kThr), 0, stream,
                               ka);
            return;
        }
    }
    // fp32 (tiny widths) computes head-wise maps densely: their zero blocks add nothing
    launch_kv<T, DH, false, BIAS, KN>(ka, ka.rows, gsz, stream);
}

template <typename T, int DH>
static void launch_translate_dh(const KVArgs& ka, int gsz, bool headwise, bool bias, bool kn, hipStream_t stream) {
    if (bias) {
        if (kn) launch_translate_group<T, DH, true, true>(ka, gsz, headwise, stream);
        else launch_translate_group<T, DH, true, false>(ka, gsz, headwise, stream);
    } else {
        if (kn) launch_translate_group<T, DH, false, true>(ka, gsz, headwise, stream);
        else launch_translate_group<T, DH, false, false>(ka, gsz, headwise, stream);
    }
}

template <typename T>
static rf_status launch_translate(const rf_translate_weights* w, int32_t n_layers, const void* const* src_k,
                                  const void* const* src_v, int64_t ld_src, int64_t t0, int64_t t1, int64_t pos0,
                                  const rf_cache_desc* cache, const rf_cache_layout_t& L, void* const* kc,
                                  void* const* vc, const int32_t* table, int64_t n_table, const float* rope,
                                  hipStream_t stream) {
    const int64_t rows = t1 - t0;
    const bool bias = w->b_k != nullptr;
    for (int l0 = 0; l0 < n_layers; l0 += kMaxGroup) {
        const int gsz = std::min(kMaxGroup, n_layers - l0);
        KVArgs ka{};
        ka.psum = nullptr; ka.ps_slot = 0; ka.n_ps = 0;
        ka.d = w->d_in; ka.kvw = w->n_kv_heads * w->head_dim; ka.eps = 0.f;
        ka.tok_tiles = (int)ceil_div(rows, kTT);
        ka.rows = rows; ka.t0 = t0; ka.pos0 = pos0; ka.rope = rope;
        ka.paged = cache->layout == RF_LAYOUT_PAGED; ka.block_size = cache->block_size;
        ka.stride_block = L.stride_block; ka.stride_head = L.stride_head; ka.stride_token = L.stride_token;
        ka.n_blocks = L.n_blocks; ka.block_table = table; ka.n_table_blocks = n_table;
        ka.ld_in = ld_src;
        ka.kn_eps = w->k_norm_eps;
        for (int g = 0; g < gsz; ++g) {
            ka.in_k[g] = src_k[l0 + g]; ka.in_v[g] = src_v[l0 + g];
            ka.kn[g] = w->k_norm ? w->k_norm[l0 + g] : nullptr;
            ka.bk[g] = bias ? w->b_k[l0 + g] : nullptr; ka.bv[g] = bias ? w->b_v[l0 + g] : nullptr;
            ka.Wk[g] = w->T_k[l0 + g]; ka.Wv[g] = w->T_v[l0 + g];
            ka.kc[g] = kc[l0 + g]; ka.vc[g] = vc[l0 + g];
        }
        const bool hw = w->headwise != 0, kn = w->k_norm != nullptr;
        if (w->head_dim == 128) launch_translate_dh<T, 128>(ka, gsz, hw, bias, kn, stream);
        else launch_translate_dh<T, 64>(ka, gsz, hw, bias, kn, stream);
        const rf_status st = check_launch("rf_translate: kernel");
        if (st != RF_OK) return st;
    }
    return RF_OK;
}

}  // namespace rf

using namespace rf;

extern "C" {

rf_status rf_rope_table(double base, int32_t head_dim, int64_t n_pos, float* d_table, void* stream) {
    clear_error();
    RF_REQUIRE(d_table, RF_ERR_INVALID_ARG, "rf_rope_table: null table");
    RF_REQUIRE(head_dim > 0 && head_dim % 2 == 0, RF_ERR_INVALID_ARG, "rf_rope_table: head_dim must be even and > 0");
    RF_REQUIRE(n_pos >= 0, RF_ERR_INVALID_ARG, "rf_rope_table: n_pos must be >= 0");
    RF_REQUIRE(base > 0 && isfinite(base), RF_ERR_INVALID_ARG, "rf_rope_table: base must be finite and > 0");
    const int64_t n = n_pos * (head_dim / 2);
    if (n == 0) return RF_OK;
    hipLaunchKernelGGL(k_rope_table, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, (hipStream_t)stream,
                       base, head_dim, (int64_t)0, n_pos, d_table);
    return check_launch("rf_rope_table");
}

size_t rf_rope_workspace_bytes(int32_t head_dim, int64_t n_tokens) {
    if (head_dim <= 0 || n_tokens < 0) return 0;
    return rope_ws_bytes(head_dim, n_tokens);
}

rf_status rf_pack_weights(rf_dtype dtype, int64_t rows, int64_t cols, const void* d_src, int64_t ld_src,
                          int32_t rope_head_dim, void* d_dst, void* stream) {
    clear_error();
    RF_REQUIRE(dtype == RF_BF16 || dtype == RF_F32, RF_ERR_UNSUPPORTED,
               "rf_pack_weights: the source must be BF16 or F32");
    RF_REQUIRE(rows >= 0 && rows % 256 == 0 && cols >= 0 && cols % 64 == 0, RF_ERR_UNSUPPORTED,
               "rf_pack_weights: rows must be a multiple of 256 and cols a multiple of 64");
    RF_REQUIRE(rope_head_dim == 0 || rope_head_dim == 64 || rope_head_dim == 128, RF_ERR_UNSUPPORTED,
               "rf_pack_weights: rope_head_dim must be 0, 64 or 128");
    RF_REQUIRE(rows <= (1 << 16) && cols <= (1 << 16), RF_ERR_UNSUPPORTED, "rf_pack_weights: rows and cols must be <= 65536");
    if (rows == 0 || cols == 0) return RF_OK;
    RF_REQUIRE(d_src && d_dst, RF_ERR_INVALID_ARG, "rf_pack_weights: null pointer argument");
    RF_REQUIRE(ld_src >= cols && ld_src % 8 == 0 && aligned(d_src, 16) && aligned(d_dst, 16), RF_ERR_INVALID_ARG,
               "rf_pack_weights: source rows must be >= cols long with a stride of 8 elements, 16-byte aligned");
    const int64_t n_chunks = rows * cols / 8;
    const dim3 grid((unsigned)ceil_div(n_chunks, 256));
    if (dtype == RF_BF16)
        hipLaunchKernelGGL(k_pack_weights<bf16_t>, grid, dim3(256), 0, (hipStream_t)stream, (const bf16_t*)d_src,
                           ld_src, cols, rope_head_dim, n_chunks, (bf16_t*)d_dst);
    else
        hipLaunchKernelGGL(k_pack_weights<float>, grid, dim3(256), 0, (hipStream_t)stream, (const float*)d_src,
                           ld_src, cols, rope_head_dim, n_chunks, (bf16_t*)d_dst);
    return check_launch("rf_pack_weights");
}

rf_status rf_quantize_map(int64_t rows, int64_t cols, const float* d_W, int64_t ld, void* d_q, float* d_scale,
                          void* stream) {
    clear_error();
    RF_REQUIRE(rows >= 0 && rows % 256 == 0 && cols >= 0 && cols % 64 == 0, RF_ERR_UNSUPPORTED,
               "rf_quantize_map: rows must be a multiple of 256 and cols a multiple of 64");
    RF_REQUIRE(rows <= (1 << 16) && cols <= (1 << 16), RF_ERR_UNSUPPORTED, "rf_quantize_map: rows and cols must be <= 65536");
    if (rows == 0 || cols == 0) return RF_OK;
    RF_REQUIRE(d_W && d_q && d_scale, RF_ERR_INVALID_ARG, "rf_quantize_map: null pointer argument");
    RF_REQUIRE(ld >= cols && ld % 4 == 0 && aligned(d_W, 16) && aligned(d_q, 16) && aligned(d_scale, 16),
               RF_ERR_INVALID_ARG, "rf_quantize_map: rows must be >= cols long with a stride of 4 floats; buffers 16-byte aligned");
    hipLaunchKernelGGL(k_quantize_map, dim3((unsigned)rows), dim3(256), 0, (hipStream_t)stream, d_W, ld, cols,
                       (int8_t*)d_q, d_scale);
    return check_launch("rf_quantize_map");
}

size_t rf_fill_workspace_bytes(const rf_fill_weights* w, int64_t max_rows) {
    if (!w || w->d <= 0 || w->d % kFT != 0 || max_rows < 0 || !valid_dtype(w->dtype)) return 0;
    return slot_bytes(w, max_rows);
}

}  // extern "C"

namespace rf {
// Host checks shared by rf_fill and rf_fill_streamed ("what" names the entry point).  Sets
// *nothing_to_do for an empty request; ws_need is the workspace the launch needs.
// The table a fill reads: the caller's (positions from 0), or -- with none given -- the table of
// the call's positions pos0 + t0 .. pos0 + t1 - 1 built at the end of the workspace, which the
// kernels then index from the call's first token (pos0 -> -t0); the workspace left for the rest
// shrinks by the table.
static rf_status prepare_rope(const float* d_rope, double base, int32_t head_dim, int64_t pos0, int64_t t0,
                              int64_t t1, void* ws, size_t& ws_bytes, const float*& rope, int64_t& pos0_eff,
                              hipStream_t stream) {
    rope = d_rope;
    pos0_eff = pos0;
    if (d_rope) return RF_OK;
    const size_t tb = rope_ws_bytes(head_dim, t1 - t0);
    const size_t off = (ws_bytes - tb) / 256 * 256;
    float* tab = (float*)((char*)ws + off);
    ws_bytes = off;
    const int64_t n = (t1 - t0) * (head_dim / 2);
    if (n > 0)
        hipLaunchKernelGGL(k_rope_table, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, stream, base, head_dim,
                           pos0 + t0, t1 - t0, tab);
    rope = tab;
    pos0_eff = -t0;
    return check_launch("rope table in the workspace");
}

static rf_status check_fill(const char* what, const rf_fill_weights* w, int32_t n_layers, const void* d_X,
                            int64_t ldx, int64_t t0, int64_t t1, int64_t pos0, const rf_cache_desc* cache,
                            void* const* k_cache, void* const* v_cache, const int32_t* d_block_table,
                            int64_t n_table_blocks, const float* d_rope, int64_t rope_len, const void* d_ws,
                            size_t ws_bytes, size_t ws_need, rf_cache_layout_t& L, bool& nothing_to_do) {
    const std::string fn = what;
    nothing_to_do = false;
    RF_REQUIRE(w && cache, RF_ERR_INVALID_ARG, fn + ": null weights or cache descriptor");
    RF_REQUIRE(n_layers >= 0, RF_ERR_INVALID_ARG, fn + ": n_layers must be >= 0");
    RF_REQUIRE(t0 >= 0 && t1 >= t0 && pos0 >= 0, RF_ERR_INVALID_ARG, fn + ": need 0 <= t0 <= t1 and pos0 >= 0");
    RF_REQUIRE(valid_dtype(w->dtype), RF_ERR_INVALID_ARG, fn + ": bad dtype");
    RF_REQUIRE(cache->dtype == w->dtype, RF_ERR_UNSUPPORTED, fn + ": cache dtype must equal the weights' dtype");
    RF_REQUIRE(w->d > 0 && w->d % kFT == 0, RF_ERR_UNSUPPORTED, fn + ": d must be a positive multiple of 256");
    RF_REQUIRE(w->head_dim == 64 || w->head_dim == 128, RF_ERR_UNSUPPORTED, fn + ": head_dim must be 64 or 128");
    RF_REQUIRE(w->n_kv_heads > 0 && (w->n_kv_heads * w->head_dim) % kFT == 0, RF_ERR_UNSUPPORTED,
               fn + ": n_kv_heads*head_dim must be a positive multiple of 256");
    RF_REQUIRE(cache->n_kv_heads == w->n_kv_heads && cache->head_dim == w->head_dim, RF_ERR_INVALID_ARG,
               fn + ": cache heads/head_dim differ from the weights'");
    RF_REQUIRE(w->rms_eps >= 0.f && isfinite(w->rms_eps), RF_ERR_INVALID_ARG, fn + ": rms_eps must be finite and >= 0");
    RF_REQUIRE(!w->k_norm || (w->k_norm_eps >= 0.f && isfinite(w->k_norm_eps)), RF_ERR_INVALID_ARG,
               fn + ": k_norm_eps must be finite and >= 0");
    RF_REQUIRE(!w->map_scale || w->dtype == RF_BF16, RF_ERR_UNSUPPORTED, fn + ": int8 maps need BF16 weights");
    rf_status st = rf_cache_layout(cache, &L);
    if (st != RF_OK) return st;
    if (n_layers == 0 || t1 == t0) {
        nothing_to_do = true;
        return RF_OK;
    }
    RF_REQUIRE(d_X && w->W_map && w->b_map && w->gamma && w->W_k && w->W_v && k_cache && v_cache && d_ws,
               RF_ERR_INVALID_ARG, fn + ": null pointer argument");
    RF_REQUIRE(d_rope || (w->rope_base > 0 && isfinite(w->rope_base)), RF_ERR_INVALID_ARG,
               fn + ": without a rope table the weights' rope_base must be finite and > 0");
    const size_t eb = elem_bytes(w->dtype);
    RF_REQUIRE(ldx >= w->d && (ldx * (int64_t)eb) % 16 == 0 && aligned(d_X, 16), RF_ERR_INVALID_ARG,
               fn + ": X rows must be >= d long, 16-byte aligned with a 16-byte multiple stride");
    RF_REQUIRE(ldx <= (1 << 21) && w->d <= (1 << 16), RF_ERR_UNSUPPORTED,
               fn + ": ldx must be <= 2^21 and d <= 65536 (32-bit tile offsets)");
    for (int l = 0; l < n_layers; ++l) {
        RF_REQUIRE(w->W_map[l] && w->b_map[l] && w->gamma[l] && w->W_k[l] && w->W_v[l] && k_cache[l] && v_cache[l],
                   RF_ERR_INVALID_ARG, fn + ": null per-layer pointer");
        RF_REQUIRE(aligned(w->W_map[l], 16) && aligned(w->W_k[l], 16) && aligned(w->W_v[l], 16) &&
                       aligned(w->b_map[l], 16) && aligned(w->gamma[l], 16) && aligned(k_cache[l], 16) &&
                       aligned(v_cache[l], 16),
                   RF_ERR_INVALID_ARG, fn + ": per-layer buffers must be 16-byte aligned");
        if (w->k_norm)
            RF_REQUIRE(w->k_norm[l] && aligned(w->k_norm[l], 16), RF_ERR_INVALID_ARG,
                       fn + ": key norm weights must be non-null and 16-byte aligned");
        if (w->map_scale)
            RF_REQUIRE(w->map_scale[l] && aligned(w->map_scale[l], 16), RF_ERR_INVALID_ARG,
                       fn + ": int8 map scales must be non-null and 16-byte aligned");
    }
    RF_REQUIRE(aligned(d_rope, 16) && aligned(d_ws, 256), RF_ERR_INVALID_ARG,
               fn + ": rope table must be 16-byte and workspace 256-byte aligned");
    if (d_rope) RF_REQUIRE(pos0 + t1 <= rope_len, RF_ERR_INVALID_ARG, fn + ": rope table shorter than pos0 + t1");
    if (cache->layout == RF_LAYOUT_PAGED) {
        RF_REQUIRE(d_block_table, RF_ERR_INVALID_ARG, fn + ": paged cache needs a block table");
        RF_REQUIRE(ceil_div(t1, cache->block_size) <= n_table_blocks, RF_ERR_INVALID_ARG,
                   fn + ": block table shorter than ceil(t1 / block_size)");
    } else {
        RF_REQUIRE(t1 <= cache->max_tokens, RF_ERR_INVALID_ARG, fn + ": t1 exceeds the cache's max_tokens");
    }
    const size_t tab = d_rope ? 0 : rope_ws_bytes(w->head_dim, t1 - t0);
    RF_REQUIRE(ws_bytes >= ws_need + tab, RF_ERR_WORKSPACE,
               fn + (d_rope ? ": workspace too small" : ": workspace too small (with the rope table it builds)"));
    return RF_OK;
}

// The maps of a streamed fill, layers_per_slot layers per ring slot: copy chunk c into slot
// c % ring_slots on copy_stream once the fill of chunk c - ring_slots has released the slot,
// and fill chunk c on stream once its copy has landed, over the whole token range in steps of
// ``rows_per_fill`` tokens (each map crosses the host link once per call, however long the
// prompt).  The first copy also waits for all
// work enqueued on stream before the call, so back-to-back calls (a chunked prompt) never
// overwrite a slot an earlier call's fill still reads.  The events only order the two
// streams; they are released when the work they mark completes.
template <typename T>
static rf_status launch_fill_streamed(const rf_fill_weights* w, int32_t n_layers, const void* X, int64_t ldx,
                                      int64_t t0, int64_t t1, int64_t pos0, const rf_cache_desc* cache,
                                      const rf_cache_layout_t& L, void* const* kc, void* const* vc,
                                      const int32_t* table, int64_t n_table, const float* rope, void* ws,
                                      size_t ws_bytes, void* ring, int32_t ring_slots, int32_t per_slot,
                                      int64_t rows_per_fill, hipStream_t stream, hipStream_t copy_stream) {
    const size_t map_bytes = (size_t)w->d * w->d * (w->map_scale ? 1 : sizeof(T));
    std::vector<hipEvent_t> copied(ring_slots, nullptr), freed(ring_slots, nullptr);
    rf_status st = RF_OK;
    auto destroy = [&]() {
        for (auto& e : copied)
            if (e) (void)hipEventDestroy(e);
        for (auto& e : freed)
            if (e) (void)hipEventDestroy(e);
    };
    for (int i = 0; i < ring_slots; ++i) {
        if (hipEventCreateWithFlags(&copied[i], hipEventDisableTiming) != hipSuccess ||
            hipEventCreateWithFlags(&freed[i], hipEventDisableTiming) != hipSuccess) {
            destroy();
            return fail(RF_ERR_HIP, "rf_fill_streamed: event creation failed");
        }
    }
    // The ring's slots may still be read by fills an earlier call (or any other work) left on
    // ``stream``: no copy of this call starts before ``stream`` has reached this point.
    hipEvent_t entry = nullptr;
    if (hipEventCreateWithFlags(&entry, hipEventDisableTiming) != hipSuccess) {
        destroy();
        return fail(RF_ERR_HIP, "rf_fill_streamed: event creation failed");
    }
    hipError_t e0 = hipEventRecord(entry, stream);
    if (e0 == hipSuccess) e0 = hipStreamWaitEvent(copy_stream, entry, 0);
    (void)hipEventDestroy(entry);
    if (e0 != hipSuccess) {
        destroy();
        return fail(RF_ERR_HIP, std::string("rf_fill_streamed: stream ordering failed: ") + hipGetErrorString(e0));
    }
    const void* maps[kMaxGroup];
    rf_fill_weights cw = *w;
    cw.W_map = maps;
    const int n_chunks = (int)ceil_div(n_layers, per_slot);
    for (int c = 0; c < n_chunks && st == RF_OK; ++c) {
        const int slot = c % ring_slots;
        const int l0 = c * per_slot, gsz = std::min(per_slot, n_layers - l0);
        char* base = (char*)ring + (size_t)slot * per_slot * map_bytes;
        hipError_t e = hipSuccess;
        if (c >= ring_slots) e = hipStreamWaitEvent(copy_stream, freed[slot], 0);
        for (int g = 0; g < gsz && e == hipSuccess; ++g) {
            maps[g] = base + (size_t)g * map_bytes;
            e = hipMemcpyAsync((void*)maps[g], w->W_map[l0 + g], map_bytes, hipMemcpyHostToDevice, copy_stream);
        }
        if (e == hipSuccess) e = hipEventRecord(copied[slot], copy_stream);
        if (e == hipSuccess) e = hipStreamWaitEvent(stream, copied[slot], 0);
        if (e != hipSuccess) {
            st = fail(RF_ERR_HIP, std::string("rf_fill_streamed: copy scheduling failed: ") + hipGetErrorString(e));
            break;
        }
        cw.b_map = w->b_map + l0; cw.gamma = w->gamma + l0; cw.W_k = w->W_k + l0; cw.W_v = w->W_v + l0;
        cw.k_norm = w->k_norm ? w->k_norm + l0 : nullptr;
        cw.map_scale = w->map_scale ? w->map_scale + l0 : nullptr;
        for (int64_t r0 = t0; r0 < t1 && st == RF_OK; r0 += rows_per_fill) {
            const int64_t r1 = std::min(t1, r0 + rows_per_fill);
            st = launch_fill<T>(&cw, gsz, (const T*)X + (r0 - t0) * ldx, ldx, r0, r1, pos0, cache, L, kc + l0, vc + l0,
                                table, n_table, rope, ws, ws_bytes, stream);
        }
        if (st == RF_OK && hipEventRecord(freed[slot], stream) != hipSuccess)
            st = fail(RF_ERR_HIP, "rf_fill_streamed: event record failed");
    }
    destroy();
    return st;
}
}  // namespace rf

namespace rf {
// Workspace of rf_fill_static: a file-scope device array (one per GPU the library runs on, held
// until the process ends).  Host code uses its device address, taken once per device with
// hipGetSymbolAddress; the array's name is not a device address on the host.
constexpr size_t kStaticScratchBytes = (size_t)RF_FILL_STATIC_SCRATCH_MB << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mutex;
static void* g_scratch_ptr[kMaxDevices];

// The current device's address of ``scratch`` (taken on the first call on that device).
static rf_status static_scratch(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(RF_ERR_HIP, std::string("rf_fill_static: hipGetDevice: ") + hipGetErrorString(e));
    RF_REQUIRE(dev >= 0 && dev < kMaxDevices, RF_ERR_UNSUPPORTED, "rf_fill_static: device index above 63");
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(RF_ERR_HIP, std::string("rf_fill_static: hipGetSymbolAddress: ") + hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return RF_OK;
}
}  // namespace rf

extern "C" {


size_t rf_fill_composed_workspace_bytes(const rf_fill_composed_weights* w, int64_t max_rows) {
    if (!w || w->d <= 0 || w->d % kFT != 0 || max_rows < 0) return 0;
    return composed_slot_bytes(w, max_rows);
}

rf_status rf_fill_composed(const rf_fill_composed_weights* w, int32_t n_layers, const void* d_X, int64_t ldx,
                           int64_t t0, int64_t t1, int64_t pos0, const rf_cache_desc* cache, void* const* k_cache,
                           void* const* v_cache, const int32_t* d_block_table, int64_t n_table_blocks,
                           const float* d_rope, int64_t rope_len, void* d_ws, size_t ws_bytes, void* stream) {
    clear_error();
    RF_REQUIRE(w && cache, RF_ERR_INVALID_ARG, "rf_fill_composed: null weights or cache descriptor");
    // the shared checks, on the composed weights seen through the fill's descriptor
    rf_fill_weights fw{};
    fw.d = w->d; fw.n_kv_heads = w->n_kv_heads; fw.head_dim = w->head_dim; fw.rms_eps = w->rms_eps; fw.dtype = RF_BF16;
    fw.W_map = w->T; fw.b_map = w->q; fw.gamma = w->c_k; fw.W_k = w->M_k; fw.W_v = w->M_v;
    fw.k_norm = w->k_norm; fw.k_norm_eps = w->k_norm_eps; fw.rope_base = w->rope_base;
    rf_cache_layout_t L;
    bool none;
    const size_t need = (w->d > 0 && w->d % kFT == 0 && t1 >= t0) ? composed_slot_bytes(w, t1 - t0) : 0;
    rf_status st = check_fill("rf_fill_composed", &fw, n_layers, d_X, ldx, t0, t1, pos0, cache, k_cache, v_cache,
                              d_block_table, n_table_blocks, d_rope, rope_len, d_ws, ws_bytes, need, L, none);
    if (st != RF_OK || none) return st;
    RF_REQUIRE(w->c_v, RF_ERR_INVALID_ARG, "rf_fill_composed: null value intercepts");
    for (int l = 0; l < n_layers; ++l)
        RF_REQUIRE(w->c_v[l] && aligned(w->c_v[l], 16), RF_ERR_INVALID_ARG,
                   "rf_fill_composed: per-layer intercepts must be non-null and 16-byte aligned");
    size_t wsb = ws_bytes;
    const float* rope = nullptr;
    int64_t p0e = pos0;
    st = prepare_rope(d_rope, w->rope_base, w->head_dim, pos0, t0, t1, d_ws, wsb, rope, p0e, (hipStream_t)stream);
    if (st != RF_OK) return st;
    return launch_fill_composed(w, n_layers, d_X, ldx, t0, t1, p0e, cache, L, k_cache, v_cache, d_block_table,
                                n_table_blocks, rope, d_ws, wsb, (hipStream_t)stream);
}

size_t rf_fill_static_scratch_bytes(void) { return rf::kStaticScratchBytes; }

rf_status rf_fill_static(const rf_fill_weights* w, int32_t n_layers, const void* d_X, int64_t ldx, int64_t t0,
                         int64_t t1, int64_t pos0, const rf_cache_desc* cache, void* const* k_cache,
                         void* const* v_cache, const int32_t* d_block_table, int64_t n_table_blocks,
                         const float* d_rope, int64_t rope_len, void* stream) {
    clear_error();
    const size_t need = (w && w->d > 0 && w->d % kFT == 0 && t1 >= t0) ? slot_bytes(w, t1 - t0) : 0;
    const size_t tab = (w && !d_rope && w->head_dim > 0 && t1 >= t0) ? rope_ws_bytes(w->head_dim, t1 - t0) : 0;
    RF_REQUIRE(need + tab <= kStaticScratchBytes, RF_ERR_UNSUPPORTED,
               "rf_fill_static: one layer of " + std::to_string(t1 - t0) + " rows needs " + std::to_string(need + tab) +
                   " bytes of scratch; the static buffer holds " + std::to_string(kStaticScratchBytes) +
                   " (fill fewer rows per call)");
    rf_cache_layout_t L;
    bool none;
    // the scratch pointer is validated below; check everything else first, against a stand-in
    const void* probe = (const void*)(uintptr_t)256;
    rf_status st = check_fill("rf_fill_static", w, n_layers, d_X, ldx, t0, t1, pos0, cache, k_cache, v_cache,
                              d_block_table, n_table_blocks, d_rope, rope_len, probe, kStaticScratchBytes, need, L,
                              none);
    if (st != RF_OK || none) return st;
    void* ws = nullptr;
    st = static_scratch(&ws);
    if (st != RF_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    size_t wsb = kStaticScratchBytes;
    const float* rope = nullptr;
    int64_t p0e = pos0;
    st = prepare_rope(d_rope, w->rope_base, w->head_dim, pos0, t0, t1, ws, wsb, rope, p0e, s);
    if (st != RF_OK) return st;
    if (w->dtype == RF_BF16)
        return launch_fill<bf16_t>(w, n_layers, d_X, ldx, t0, t1, p0e, cache, L, k_cache, v_cache, d_block_table,
                                   n_table_blocks, rope, ws, wsb, s);
    return launch_fill<float>(w, n_layers, d_X, ldx, t0, t1, p0e, cache, L, k_cache, v_cache, d_block_table,
                              n_table_blocks, rope, ws, wsb, s);
}

rf_status rf_fill(const rf_fill_weights* w, int32_t n_layers, const void* d_X, int64_t ldx,
                  int64_t t0, int64_t t1, int64_t pos0, const rf_cache_desc* cache,
                  void* const* k_cache, void* const* v_cache, const int32_t* d_block_table,
                  int64_t n_table_blocks, const float* d_rope, int64_t rope_len, void* d_ws,
                  size_t ws_bytes, void* stream) {
    clear_error();
    rf_cache_layout_t L;
    bool none;
    const size_t need = (w && w->d > 0 && w->d % kFT == 0 && t1 >= t0) ? slot_bytes(w, t1 - t0) : 0;
    const rf_status st = check_fill("rf_fill", w, n_layers, d_X, ldx, t0, t1, pos0, cache, k_cache, v_cache,
                                    d_block_table, n_table_blocks, d_rope, rope_len, d_ws, ws_bytes, need, L, none);
    if (st != RF_OK || none) return st;
    hipStream_t s = (hipStream_t)stream;
    size_t wsb = ws_bytes;
    const float* rope = nullptr;
    int64_t p0e = pos0;
    rf_status rs = prepare_rope(d_rope, w->rope_base, w->head_dim, pos0, t0, t1, d_ws, wsb, rope, p0e, s);
    if (rs != RF_OK) return rs;
    if (w->dtype == RF_BF16)
        return launch_fill<bf16_t>(w, n_layers, d_X, ldx, t0, t1, p0e, cache, L, k_cache, v_cache, d_block_table,
                                   n_table_blocks, rope, d_ws, wsb, s);
    return launch_fill<float>(w, n_layers, d_X, ldx, t0, t1, p0e, cache, L, k_cache, v_cache, d_block_table,
                              n_table_blocks, rope, d_ws, wsb, s);
}

size_t rf_fill_streamed_ring_bytes(const rf_fill_weights* w, int32_t ring_slots, int32_t layers_per_slot) {
    if (!w || w->d <= 0 || w->d % kFT != 0 || !valid_dtype(w->dtype) || ring_slots < 1 || layers_per_slot < 1)
        return 0;
    return (size_t)ring_slots * layers_per_slot * w->d * w->d * (w->map_scale ? 1 : elem_bytes(w->dtype));
}

rf_status rf_fill_streamed(const rf_fill_weights* w, int32_t n_layers, const void* d_X, int64_t ldx,
                           int64_t t0, int64_t t1, int64_t pos0, const rf_cache_desc* cache,
                           void* const* k_cache, void* const* v_cache, const int32_t* d_block_table,
                           int64_t n_table_blocks, const float* d_rope, int64_t rope_len, void* d_ws,
                           size_t ws_bytes, void* d_ring, size_t ring_bytes, int32_t ring_slots,
                           int32_t layers_per_slot, int64_t rows_per_fill, void* stream, void* copy_stream) {
    clear_error();
    RF_REQUIRE(ring_slots >= 1 && layers_per_slot >= 1 && layers_per_slot <= kMaxGroup, RF_ERR_INVALID_ARG,
               "rf_fill_streamed: need ring_slots >= 1 and 1 <= layers_per_slot <= 32");
    RF_REQUIRE(rows_per_fill >= 0, RF_ERR_INVALID_ARG, "rf_fill_streamed: rows_per_fill must be >= 0");
    const int64_t rpf = rows_per_fill == 0 || rows_per_fill > t1 - t0 ? std::max<int64_t>(t1 - t0, 1) : rows_per_fill;
    rf_cache_layout_t L;
    bool none;
    const size_t need = (w && w->d > 0 && w->d % kFT == 0 && t1 >= t0) ? slot_bytes(w, rpf) * layers_per_slot : 0;
    rf_status st = check_fill("rf_fill_streamed", w, n_layers, d_X, ldx, t0, t1, pos0, cache, k_cache, v_cache,
                              d_block_table, n_table_blocks, d_rope, rope_len, d_ws, ws_bytes, need, L, none);
    if (st != RF_OK || none) return st;
    RF_REQUIRE(copy_stream && copy_stream != stream, RF_ERR_INVALID_ARG,
               "rf_fill_streamed: the copies need a stream of their own");
    RF_REQUIRE(d_ring && aligned(d_ring, 256), RF_ERR_INVALID_ARG, "rf_fill_streamed: ring must be 256-byte aligned");
    RF_REQUIRE(ring_bytes >= rf_fill_streamed_ring_bytes(w, ring_slots, layers_per_slot), RF_ERR_WORKSPACE,
               "rf_fill_streamed: ring too small");
    hipStream_t s = (hipStream_t)stream, cs = (hipStream_t)copy_stream;
    size_t wsb = ws_bytes;
    const float* rope = nullptr;
    int64_t p0e = pos0;
    st = prepare_rope(d_rope, w->rope_base, w->head_dim, pos0, t0, t1, d_ws, wsb, rope, p0e, s);
    if (st != RF_OK) return st;
    if (w->dtype == RF_BF16)
        return launch_fill_streamed<bf16_t>(w, n_layers, d_X, ldx, t0, t1, p0e, cache, L, k_cache, v_cache,
                                            d_block_table, n_table_blocks, rope, d_ws, wsb, d_ring, ring_slots,
                                            layers_per_slot, rpf, s, cs);
    return launch_fill_streamed<float>(w, n_layers, d_X, ldx, t0, t1, p0e, cache, L, k_cache, v_cache,
                                       d_block_table, n_table_blocks, rope, d_ws, wsb, d_ring, ring_slots,
                                       layers_per_slot, rpf, s, cs);
}

rf_status rf_translate(const rf_translate_weights* w, int32_t n_layers, const void* const* d_src_k,
                       const void* const* d_src_v, int64_t ld_src, int64_t t0, int64_t t1, int64_t pos0,
                       const rf_cache_desc* cache, void* const* k_cache, void* const* v_cache,
                       const int32_t* d_block_table, int64_t n_table_blocks, const float* d_rope,
                       int64_t rope_len, void* stream) {
    clear_error();
    RF_REQUIRE(w && cache, RF_ERR_INVALID_ARG, "rf_translate: null weights or cache descriptor");
    RF_REQUIRE(n_layers >= 0, RF_ERR_INVALID_ARG, "rf_translate: n_layers must be >= 0");
    RF_REQUIRE(t0 >= 0 && t1 >= t0 && pos0 >= 0, RF_ERR_INVALID_ARG, "rf_translate: need 0 <= t0 <= t1 and pos0 >= 0");
    RF_REQUIRE(valid_dtype(w->dtype), RF_ERR_INVALID_ARG, "rf_translate: bad dtype");
    RF_REQUIRE(cache->dtype == w->dtype, RF_ERR_UNSUPPORTED, "rf_translate: cache dtype must equal the maps' dtype");
    const int din_step = w->dtype == RF_BF16 ? 128 : 64;
    RF_REQUIRE(w->d_in > 0 && w->d_in % din_step == 0 && w->d_in <= (1 << 16), RF_ERR_UNSUPPORTED,
               "rf_translate: d_in must be a positive multiple of 128 (BF16) or 64 (F32), at most 65536");
    RF_REQUIRE(w->head_dim == 64 || w->head_dim == 128, RF_ERR_UNSUPPORTED, "rf_translate: head_dim must be 64 or 128");
    RF_REQUIRE(w->n_kv_heads > 0 && (w->n_kv_heads * w->head_dim) % kFT == 0, RF_ERR_UNSUPPORTED,
               "rf_translate: n_kv_heads*head_dim must be a positive multiple of 256");
    RF_REQUIRE(cache->n_kv_heads == w->n_kv_heads && cache->head_dim == w->head_dim, RF_ERR_INVALID_ARG,
               "rf_translate: cache heads/head_dim differ from the maps'");
    RF_REQUIRE((w->b_k == nullptr) == (w->b_v == nullptr), RF_ERR_INVALID_ARG,
               "rf_translate: b_k and b_v must both be given or both be NULL");
    RF_REQUIRE(w->headwise == 0 || w->headwise == 1, RF_ERR_INVALID_ARG, "rf_translate: headwise must be 0 or 1");
    RF_REQUIRE(!w->k_norm || (w->k_norm_eps >= 0.f && isfinite(w->k_norm_eps)), RF_ERR_INVALID_ARG,
               "rf_translate: k_norm_eps must be finite and >= 0");
    RF_REQUIRE(!w->headwise || w->d_in % (w->n_kv_heads * w->head_dim) == 0, RF_ERR_UNSUPPORTED,
               "rf_translate: head-wise maps need d_in = nu * n_kv_heads * head_dim (source heads as the target's)");
    rf_cache_layout_t L;
    rf_status st = rf_cache_layout(cache, &L);
    if (st != RF_OK) return st;
    if (n_layers == 0 || t1 == t0) return RF_OK;
    RF_REQUIRE(d_src_k && d_src_v && w->T_k && w->T_v && k_cache && v_cache, RF_ERR_INVALID_ARG,
               "rf_translate: null pointer argument");
    const size_t eb = elem_bytes(w->dtype);
    RF_REQUIRE(ld_src >= w->d_in && (ld_src * (int64_t)eb) % 16 == 0 && ld_src <= (1 << 21), RF_ERR_INVALID_ARG,
               "rf_translate: source rows must be >= d_in long with a 16-byte multiple stride of at most 2^21 elements");
    const bool bias = w->b_k != nullptr;
    for (int l = 0; l < n_layers; ++l) {
        RF_REQUIRE(d_src_k[l] && d_src_v[l] && w->T_k[l] && w->T_v[l] && k_cache[l] && v_cache[l], RF_ERR_INVALID_ARG,
                   "rf_translate: null per-layer pointer");
        RF_REQUIRE(aligned(d_src_k[l], 16) && aligned(d_src_v[l], 16) && aligned(w->T_k[l], 16) &&
                       aligned(w->T_v[l], 16) && aligned(k_cache[l], 16) && aligned(v_cache[l], 16),
                   RF_ERR_INVALID_ARG, "rf_translate: per-layer buffers must be 16-byte aligned");
        if (bias)
            RF_REQUIRE(w->b_k[l] && w->b_v[l] && aligned(w->b_k[l], 16) && aligned(w->b_v[l], 16), RF_ERR_INVALID_ARG,
                       "rf_translate: intercepts must be non-null and 16-byte aligned");
        if (w->k_norm)
            RF_REQUIRE(w->k_norm[l] && aligned(w->k_norm[l], 16), RF_ERR_INVALID_ARG,
                       "rf_translate: key norm weights must be non-null and 16-byte aligned");
    }
    if (d_rope) {
        RF_REQUIRE(aligned(d_rope, 16), RF_ERR_INVALID_ARG, "rf_translate: rope table must be 16-byte aligned");
        RF_REQUIRE(pos0 + t1 <= rope_len, RF_ERR_INVALID_ARG, "rf_translate: rope table shorter than pos0 + t1");
    }
    if (cache->layout == RF_LAYOUT_PAGED) {
        RF_REQUIRE(d_block_table, RF_ERR_INVALID_ARG, "rf_translate: paged cache needs a block table");
        RF_REQUIRE(ceil_div(t1, cache->block_size) <= n_table_blocks, RF_ERR_INVALID_ARG,
                   "rf_translate: block table shorter than ceil(t1 / block_size)");
    } else {
        RF_REQUIRE(t1 <= cache->max_tokens, RF_ERR_INVALID_ARG, "rf_translate: t1 exceeds the cache's max_tokens");
    }
    hipStream_t s = (hipStream_t)stream;
    if (translate_headwise_supported(w))
        return launch_translate_headwise(w, n_layers, d_src_k, d_src_v, ld_src, t0, t1, pos0, cache, L, k_cache,
                                         v_cache, d_block_table, n_table_blocks, d_rope, s);
    if (w->dtype == RF_BF16)
        return launch_translate<bf16_t>(w, n_layers, d_src_k, d_src_v, ld_src, t0, t1, pos0, cache, L, k_cache,
                                        v_cache, d_block_table, n_table_blocks, d_rope, s);
    return launch_translate<float>(w, n_layers, d_src_k, d_src_v, ld_src, t0, t1, pos0, cache, L, k_cache, v_cache,
                                   d_block_table, n_table_blocks, d_rope, s);
}

}  // extern "C"
