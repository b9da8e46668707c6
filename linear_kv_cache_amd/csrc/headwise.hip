// Token-wise cache translators with head-wise maps (KV-Lingo page, section 3.1 "Head mixing":
// a head-wise translator maps each source head only onto the same target head, so its map is
// block-diagonal by head; section 3.2 fits it in closed form).
//
// A work-group owns one 256-feature tile of one side (keys or values) of one target layer --
// 256 / d_h heads -- and a run of tokens.  Its four waves are the four 64-row blocks of the
// tile in the packed weight order (rf_pack_weights with rope_head_dim = d_h): each wave holds
// 32 RoPE pairs of one head and keeps that head's block of the map (64 rows x d_h columns of
// each of the nu source layers) in registers for the whole run, so only the block-diagonal
// products are computed.  Tokens stream in blocks of 32 (the MFMA's N): the tile's 256 columns
// of each source layer, loaded two blocks ahead into two register sets, written to one of two
// LDS stages a block ahead, and read from LDS as MFMA fragments.  Every block issues the same
// loads in the same order (a run's last blocks re-read its last row), so the compiler's
// load-count waits keep two blocks in flight; anything the epilogue reads from memory (RoPE
// rows one block ahead, intercepts and key-norm weights for the whole run, the block table
// into LDS) is loaded before the blocks it would otherwise wait for.  Per block each wave runs
// 2 x nu x d_h / 16 v_mfma_f32_32x32x16_bf16, then the epilogue of the dense translator:
// intercept, per-head key norm, RoPE on lane-local pairs, and whole 16-byte row stores to the
// caches, staged through LDS.
#include "rf_internal.h"
#include "rf_mfma.h"
#include "rf_pipe.h"

namespace rf {

constexpr int kHwTok = 32;          // tokens per block: the MFMA's N
constexpr int kHwThr = 256;         // 4 waves
constexpr int kHwTile = 256;        // target features per work-group
constexpr int kHwMaxLayers = 32;    // target layers per launch
constexpr int kHwMaxChunk = 4096;   // tokens per work-group at most

struct HwArgs {
    int32_t kvw;             // n_kv_heads * head_dim
    int32_t tiles;           // kvw / 256
    int64_t d_in;            // nu * kvw
    int64_t rows;            // tokens t0 .. t0 + rows - 1
    int64_t t0, pos0;
    int64_t ld_src;          // elements between source rows
    int32_t chunk;           // tokens per work-group (multiple of 32)
    int32_t n_chunks;
    const float* rope;       // [pos][head_dim/2][2], or null: keys are not rotated
    int32_t paged, block_size;
    int64_t stride_block, stride_head, stride_token, n_blocks, n_table_blocks;
    const int32_t* block_table;
    float kn_eps;
    const bf16_t* src_k[kHwMaxLayers];
    const bf16_t* src_v[kHwMaxLayers];
    const bf16_t* Tk[kHwMaxLayers];
    const bf16_t* Tv[kHwMaxLayers];
    const float* bk[kHwMaxLayers];
    const float* bv[kHwMaxLayers];
    const float* kn[kHwMaxLayers];
    bf16_t* kc[kHwMaxLayers];
    bf16_t* vc[kHwMaxLayers];
};

template <int NU>
struct HwRing {
    static constexpr int ROWB = NU * 512;                  // staged bytes per token
    static constexpr int STAGE = kHwTok * ROWB;            // 16 KiB per source layer
    static constexpr int LW = STAGE / (kHwThr * 16);       // 16-byte loads per thread per block
    static_assert(LW * kHwThr * 16 == STAGE, "whole 16-byte pieces");
};

template <int DH, int NU, bool BIAS, bool KN>
__global__ __launch_bounds__(kHwThr) void k_translate_hw(HwArgs a) {
    using R = HwRing<NU>;
    constexpr int LW = R::LW, HALF = DH / 2;
    constexpr int NKS = DH / 16;                    // k-slices of one head per source layer
    __shared__ __attribute__((aligned(16))) char stg[2][R::STAGE];
    __shared__ __attribute__((aligned(16))) char outb[kHwTok * kHwTile * 2];
    __shared__ int64_t rbase[kHwTok];
    __shared__ float knred[4][kHwTok];
    __shared__ int32_t tabl[kHwMaxChunk + 2];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int u = xcd_order((int)blockIdx.x, (int)gridDim.x);
    const int unit = u / a.n_chunks, chunk = u - unit * a.n_chunks;
    const int g = unit / (2 * a.tiles);
    const int rem = unit - g * 2 * a.tiles;
    const bool is_k = rem < a.tiles;
    const int t = is_k ? rem : rem - a.tiles;
    const int64_t c0 = (int64_t)chunk * a.chunk;
    if (c0 >= a.rows) return;
    const int64_t crow = a.rows - c0 < a.chunk ? a.rows - c0 : a.chunk;   // tokens of this run
    const int nb = (int)ceil_div(crow, kHwTok);

    // the wave's head: its columns within the tile's 256-column block of each source layer
    const int col0 = DH == 128 ? (wave >> 1) * 128 : wave * 64;
    // map fragments: packed tile t, k-step of column (s kvw + 256 t + col0 + 16 ks), this
    // wave's 64 rows, slice, 32-row block i; 1 KiB per fragment, 16 B per lane
    u32x4 fa[2][NU][NKS];
    {
        const bf16_t* Tsel = (is_k ? a.Tk[g] : a.Tv[g]) + (int64_t)t * kHwTile * a.d_in;
#pragma unroll
        for (int s = 0; s < NU; ++s)
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const int64_t col = (int64_t)s * a.kvw + (int64_t)t * kHwTile + col0 + 16 * ks;
                const int64_t base = (col / 64) * 16384 + wave * 4096 + ((col % 64) / 16) * 1024 + lane * 8;
#pragma unroll
                for (int i = 0; i < 2; ++i) fa[i][s][ks] = *(const u32x4*)(Tsel + base + i * 512);
            }
    }
    // staged block: byte o = (wave LW + j) 1 KiB + 16 lane of a stage holds token o / ROWB,
    // source layer (o % ROWB) / 512 and 16-byte slot p = (o % 512) / 16, which holds the
    // tile's chunk p ^ (token & 15) of that layer (swizzled for conflict-free fragment reads);
    // thread (wave, lane) loads and writes exactly those pieces
    const char* src = (const char*)(is_k ? a.src_k[g] : a.src_v[g]) + ((int64_t)t * kHwTile) * 2;
    int ld_tok[LW], ld_off[LW];
#pragma unroll
    for (int j = 0; j < LW; ++j) {
        const int o = (wave * LW + j) * 1024 + lane * 16;
        const int n = o / R::ROWB, s = (o % R::ROWB) / 512, p = (o % 512) / 16;
        ld_tok[j] = n;
        ld_off[j] = s * a.kvw * 2 + ((p ^ (n & 15)) << 4);
    }
    auto gload = [&](u32x4 (&r)[LW], int b) {
        const int64_t n0 = c0 + (int64_t)b * kHwTok;
#pragma unroll
        for (int j = 0; j < LW; ++j) {
            int64_t n = n0 + ld_tok[j];
            n = n < a.rows ? n : a.rows - 1;                 // past the run: a valid row, not stored
            r[j] = *(const u32x4*)(src + n * a.ld_src * 2 + ld_off[j]);
        }
    };
    auto swrite = [&](char* stage, const u32x4 (&r)[LW]) {
#pragma unroll
        for (int j = 0; j < LW; ++j) *(u32x4*)(stage + (wave * LW + j) * 1024 + lane * 16) = r[j];
    };

    bf16_t* pool = is_k ? a.kc[g] : a.vc[g];
    const float* bsel = BIAS ? (is_k ? a.bk[g] : a.bv[g]) + (int64_t)t * kHwTile : nullptr;
    const int qp0 = wave * 32 + 4 * (lane >> 5);     // first RoPE pair of the lane (as k_fill_kv)
    // the lane's intercepts and key-norm weights, held for the run (a load in the epilogue
    // would wait for every block in flight)
    f32x4 b_lo[4], b_hi[4], g_lo[4], g_hi[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int qp = qp0 + 8 * q;
        const int fl = (qp / HALF) * DH + qp % HALF;
        b_lo[q] = b_hi[q] = g_lo[q] = g_hi[q] = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (BIAS) {
            b_lo[q] = *(const f32x4*)(bsel + fl);
            b_hi[q] = *(const f32x4*)(bsel + fl + HALF);
        }
        if constexpr (KN) {   // value tiles load them too (unused): the same loads on every tile
            g_lo[q] = *(const f32x4*)(a.kn[g] + qp % HALF);
            g_hi[q] = *(const f32x4*)(a.kn[g] + qp % HALF + HALF);
        }
    }
    const int nl = lane & 31;                        // the lane's token in a block
    const bool rot = is_k && a.rope != nullptr;
    // (cos, sin) of the lane's 16 low dims for its token of a block.  Loaded on every block and
    // every tile (value tiles and tables-less keys read the map's first bytes and discard them),
    // so each block issues the same loads and the compiler's load counts stay exact.
    const float* cs_base = a.rope ? a.rope : (const float*)(is_k ? a.Tk[g] : a.Tv[g]);
    auto rope_load = [&](f32x4 (&c01)[4], f32x4 (&c23)[4], int b) {
        int64_t n = c0 + (int64_t)b * kHwTok + nl;
        n = n < a.rows ? n : a.rows - 1;
        const float* cs_row = cs_base + (a.rope ? (a.pos0 + a.t0 + n) * (int64_t)DH : 0);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int dlo = (qp0 + 8 * q) % HALF;
            c01[q] = *(const f32x4*)(cs_row + 2 * dlo);
            c23[q] = *(const f32x4*)(cs_row + 2 * dlo + 4);
        }
    };
    // paged caches: the block-table entries of the run's tokens, read once into LDS (a table
    // load inside the stream would wait for every block in flight)
    const int64_t lb0 = a.paged ? (a.t0 + c0) / a.block_size : 0;
    if (a.paged) {
        const int64_t n_ent = (a.t0 + c0 + crow - 1) / a.block_size - lb0 + 1;
        for (int64_t i = threadIdx.x; i < n_ent; i += kHwThr)
            tabl[i] = lb0 + i < a.n_table_blocks ? a.block_table[lb0 + i] : -1;
    }
    // cache row offset of token threadIdx.x of block b, or -1 (past the run, or no cache slot)
    auto row_base = [&](int b) -> int64_t {
        const int64_t n = c0 + (int64_t)b * kHwTok + threadIdx.x;
        if (n >= a.rows) return -1;
        const int64_t tok = a.t0 + n;
        if (!a.paged) return tok * a.stride_token;
        const int32_t phys = tabl[tok / a.block_size - lb0];
        if (phys < 0 || phys >= a.n_blocks) return -1;
        return (int64_t)phys * a.stride_block + (tok % a.block_size) * a.stride_token;
    };

    u32x4 r0[LW], r1[LW];
    f32x4 ca01[4], ca23[4], cb01[4], cb23[4];

    // one block: S = stg[b & 1] holds block b, ``rn`` holds block b + 1 (loaded a block ago),
    // ``rf`` block b + 2 (in flight); ``cc`` the (cos, sin) of block b, ``cn`` gets block b + 1's
    auto step = [&](int b, char* S, char* Sn, u32x4 (&rn)[LW], u32x4 (&rf)[LW], f32x4 (&cc01)[4],
                    f32x4 (&cc23)[4], f32x4 (&cn01)[4], f32x4 (&cn23)[4]) {
        if (threadIdx.x < kHwTok) rbase[threadIdx.x] = row_base(b);
        // the next block's (cos, sin) first (their wait then covers only older loads)
        rope_load(cn01, cn23, b + 1);
        // products: B fragment = token nl, 8 columns (col0 + 16 ks + 8 (lane >> 5)) of layer s
        f32x16 acc0 = {}, acc1 = {};
#pragma unroll
        for (int s = 0; s < NU; ++s)
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const int c = (col0 >> 3) + 2 * ks + (lane >> 5);
                const u32x4 fb = *(const u32x4*)(S + nl * R::ROWB + s * 512 + ((c ^ (nl & 15)) << 4));
                acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, fa[0][s][ks]),
                                                               __builtin_bit_cast(bf16x8, fb), acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, fa[1][s][ks]),
                                                               __builtin_bit_cast(bf16x8, fb), acc1, 0, 0, 0);
            }
        // block b + 1 into the other stage (read last by block b - 1, before the last barrier),
        // then its registers take block b + 3.  Past the run the loads read the run's last row
        // and the stage write is never read: every block runs the same straight-line code.  (A
        // branch around the write let the accumulators be read too soon after the last MFMA on
        // the path that skipped it: the wait states it needs were only placed on the other.)
        swrite(Sn, rn);
        gload(rn, b + 3);
        (void)rf;
        // staged outputs: [token][feature], 16-byte chunk c of token n in slot c ^ (n & 31)
        auto stage_out = [&](int fl, const float (&o)[4]) {
            const int slot = ((fl >> 3) ^ nl) << 4;
            *(u32x2*)(outb + nl * (kHwTile * 2) + slot + (fl & 4) * 2) =
                u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
        };
        if (!is_k) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int qp = qp0 + 8 * q;
                const int fl = (qp / HALF) * DH + qp % HALF;
                float lo[4], hi[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    lo[e] = acc0[4 * q + e] + b_lo[q][e];
                    hi[e] = acc1[4 * q + e] + b_hi[q][e];
                }
                stage_out(fl, lo);
                stage_out(fl + HALF, hi);
            }
        } else {
            float kinv = 1.f;
            if constexpr (KN) {
                // the head's sum of squares: the lane's 32 values, its partner lane (lane ^ 32)
                // and, for 128-wide heads, the partner wave (wave ^ 1) through LDS
                float ss = 0.f;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float x = acc0[4 * q + e] + b_lo[q][e], y = acc1[4 * q + e] + b_hi[q][e];
                        ss += x * x + y * y;
                    }
                }
                ss += __shfl_xor(ss, 32);
                if (lane < 32) knred[wave][nl] = ss;
                __syncthreads();
                float ssh = knred[wave][nl];
                if constexpr (DH == 128) ssh += knred[wave ^ 1][nl];
                kinv = 1.0f / sqrtf(ssh * (1.0f / (float)DH) + a.kn_eps);
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int qp = qp0 + 8 * q;
                const int fl = (qp / HALF) * DH + qp % HALF;
                const float cs[4] = {rot ? cc01[q][0] : 1.f, rot ? cc01[q][2] : 1.f, rot ? cc23[q][0] : 1.f,
                                     rot ? cc23[q][2] : 1.f};
                const float sn[4] = {rot ? cc01[q][1] : 0.f, rot ? cc01[q][3] : 0.f, rot ? cc23[q][1] : 0.f,
                                     rot ? cc23[q][3] : 0.f};
                float lo[4], hi[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float x = acc0[4 * q + e] + b_lo[q][e];
                    float y = acc1[4 * q + e] + b_hi[q][e];
                    if constexpr (KN) {
                        x *= kinv * g_lo[q][e];
                        y *= kinv * g_hi[q][e];
                    }
                    lo[e] = x * cs[e] - y * sn[e];
                    hi[e] = y * cs[e] + x * sn[e];
                }
                stage_out(fl, lo);
                stage_out(fl + HALF, hi);
            }
        }
        __syncthreads();
        // whole 16-byte pieces of (token, head) rows: chunk c = features 8c .. 8c + 7
        const int c = threadIdx.x & 31;
        const int f = t * kHwTile + c * 8;
        const int64_t hoff = (int64_t)(f / DH) * a.stride_head + f % DH;
#pragma unroll
        for (int p = 0; p < kHwTok / 8; ++p) {
            const int tn = p * 8 + (threadIdx.x >> 5);
            const int64_t base = rbase[tn];
            const u32x4 v = *(const u32x4*)(outb + tn * (kHwTile * 2) + ((c ^ tn) << 4));
            if (base >= 0) *(u32x4*)(pool + base + hoff) = v;
        }
        // block b + 1's stage written, this block's stage, outputs and row offsets all read
        __syncthreads();
    };

    // prologue: block 0 in LDS; then, in the order the loop issues them, block 1, block 0's
    // (cos, sin) and block 2 in flight (the same load counts as at every later even block)
    gload(r0, 0);
    swrite(stg[0], r0);
    __builtin_amdgcn_sched_barrier(0);
    gload(r1, 1);
    __builtin_amdgcn_sched_barrier(0);
    rope_load(ca01, ca23, 0);
    __builtin_amdgcn_sched_barrier(0);
    gload(r0, 2);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    // even blocks: stage 0, the next block in r1, the one after in r0; odd blocks the other way
    // (both steps in every trip, so the loop's load counts are the same on every path)
    int b = 0;
    for (; b + 1 < nb; b += 2) {
        step(b, stg[0], stg[1], r1, r0, ca01, ca23, cb01, cb23);
        step(b + 1, stg[1], stg[0], r0, r1, cb01, cb23, ca01, ca23);
    }
    if (b < nb) step(b, stg[0], stg[1], r1, r0, ca01, ca23, cb01, cb23);
}

template <int DH, int NU>
static void launch_hw_dh_nu(const HwArgs& ha, dim3 grid, bool bias, bool kn, hipStream_t s) {
    if (bias) {
        if (kn) hipLaunchKernelGGL((k_translate_hw<DH, NU, true, true>), grid, dim3(kHwThr), 0, s, ha);
        else hipLaunchKernelGGL((k_translate_hw<DH, NU, true, false>), grid, dim3(kHwThr), 0, s, ha);
    } else {
        if (kn) hipLaunchKernelGGL((k_translate_hw<DH, NU, false, true>), grid, dim3(kHwThr), 0, s, ha);
        else hipLaunchKernelGGL((k_translate_hw<DH, NU, false, false>), grid, dim3(kHwThr), 0, s, ha);
    }
}

bool translate_headwise_supported(const rf_translate_weights* w) {
    if (w->dtype != RF_BF16 || !w->headwise) return false;
    const int64_t kvw = (int64_t)w->n_kv_heads * w->head_dim;
    const int64_t nu = w->d_in / kvw;
    // nu = 3 would hold 96 (d_h = 64) or 192 (d_h = 128) registers of map per lane: it spills
    return nu >= 1 && nu <= 2 && nu * kvw == w->d_in;
}

rf_status launch_translate_headwise(const rf_translate_weights* w, int32_t n_layers, const void* const* src_k,
                                    const void* const* src_v, int64_t ld_src, int64_t t0, int64_t t1, int64_t pos0,
                                    const rf_cache_desc* cache, const rf_cache_layout_t& L, void* const* kc,
                                    void* const* vc, const int32_t* table, int64_t n_table, const float* rope,
                                    hipStream_t stream) {
    const int64_t rows = t1 - t0;
    const int kvw = w->n_kv_heads * w->head_dim;
    const int nu = (int)(w->d_in / kvw);
    const bool bias = w->b_k != nullptr, kn = w->k_norm != nullptr;
    for (int l0 = 0; l0 < n_layers; l0 += kHwMaxLayers) {
        const int gsz = std::min(kHwMaxLayers, n_layers - l0);
        HwArgs ha{};
        ha.kvw = kvw; ha.tiles = kvw / kHwTile; ha.d_in = w->d_in;
        ha.rows = rows; ha.t0 = t0; ha.pos0 = pos0; ha.ld_src = ld_src;
        // runs of tokens: about four work-groups per CU over the launch, at least 8 blocks each
        const int64_t units = (int64_t)gsz * 2 * ha.tiles;
        const int64_t want = std::max<int64_t>(1, 1024 / units);
        int64_t chunk = ceil_div(ceil_div(rows, want), kHwTok) * kHwTok;
        chunk = std::max<int64_t>(chunk, 8 * kHwTok);
        ha.chunk = (int32_t)std::min<int64_t>(chunk, kHwMaxChunk);
        ha.n_chunks = (int32_t)ceil_div(rows, ha.chunk);
        ha.rope = rope;
        ha.paged = cache->layout == RF_LAYOUT_PAGED; ha.block_size = cache->block_size;
        ha.stride_block = L.stride_block; ha.stride_head = L.stride_head; ha.stride_token = L.stride_token;
        ha.n_blocks = L.n_blocks; ha.block_table = table; ha.n_table_blocks = n_table;
        ha.kn_eps = w->k_norm_eps;
        for (int gi = 0; gi < gsz; ++gi) {
            const int l = l0 + gi;
            ha.src_k[gi] = (const bf16_t*)src_k[l]; ha.src_v[gi] = (const bf16_t*)src_v[l];
            ha.Tk[gi] = (const bf16_t*)w->T_k[l]; ha.Tv[gi] = (const bf16_t*)w->T_v[l];
            ha.bk[gi] = bias ? w->b_k[l] : nullptr; ha.bv[gi] = bias ? w->b_v[l] : nullptr;
            ha.kn[gi] = kn ? w->k_norm[l] : nullptr;
            ha.kc[gi] = (bf16_t*)kc[l]; ha.vc[gi] = (bf16_t*)vc[l];
        }
        const dim3 grid((unsigned)(units * ha.n_chunks));
        if (w->head_dim == 128) {
            if (nu == 1) launch_hw_dh_nu<128, 1>(ha, grid, bias, kn, stream);
            else launch_hw_dh_nu<128, 2>(ha, grid, bias, kn, stream);
        } else {
            if (nu == 1) launch_hw_dh_nu<64, 1>(ha, grid, bias, kn, stream);
            else launch_hw_dh_nu<64, 2>(ha, grid, bias, kn, stream);
        }
        const rf_status st = check_launch("rf_translate: head-wise kernel");
        if (st != RF_OK) return st;
    }
    return RF_OK;
}

}  // namespace rf
