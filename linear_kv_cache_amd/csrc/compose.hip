// Composition of the fill's weights (rf_fill_compose): a filled layer's map folded into its
// own K/V projections, and the map's sum of squares as a triangular quadratic form
// (RidgeFill project page, "Method" steps 2-4: only the layer's K/V rows are written, and the
// predicted input reaches them only through its RMS and its projections).
//
// Per layer, from the packed bf16 map W ([d][d]), its intercept b, the layer's gamma and its
// packed W_k, W_v ([kvw][d], rows in RoPE-pair order):
//   A2 = [W^T | W^T]                            [d][2d] bf16, W transposed out of the packing
//   B2 = [hi | lo] of (W_k,v diag(gamma))       [2 kvw][2d] bf16, rows in the packed order
//   T  = strict upper triangle of 2 W^T W       one PipeGemm tile per 256 x 256 block on or
//                                               above the diagonal (A = B = W^T, K = d); the
//                                               diagonal of W^T W stays fp32 (in q)
//   M  = W_k,v diag(gamma) W                    M^T tiles with A = A2 rows, B = B2 rows,
//                                               K = 2d (hi and lo parts summed in fp32)
//   c  = W_k,v diag(gamma) b, q = [2 W^T b, diag(W^T W), |b|^2]   fp32
// T and M are written in the fill's packed fragment order (M keeps the RoPE-pair row order of
// W_k, W_v, so the K/V launch reads it exactly as it reads W_k, W_v).
#include <algorithm>

#include "rf_internal.h"
#include "rf_mfma.h"
#include "rf_pipe.h"

#define RF_TRY_LAUNCH(what)                   \
    do {                                      \
        rf_status _st = rf::check_launch(what); \
        if (_st != RF_OK) return _st;         \
    } while (0)

namespace rf {

constexpr int kCT = 256;   // tile

constexpr int kComposeGroup = 32;   // layers per launch at most

// Per-layer operands of the preparation launches (layer g = the launch's last grid index).
struct PrepArgs {
    const bf16_t* W[kComposeGroup];      // packed map
    const bf16_t* Wk[kComposeGroup];
    const bf16_t* Wv[kComposeGroup];
    const float* gamma[kComposeGroup];
    const float* b[kComposeGroup];
    bf16_t* A2[kComposeGroup];
    bf16_t* B2[kComposeGroup];
    float* ck[kComposeGroup];
    float* cv[kComposeGroup];
    float* q[kComposeGroup];
};

// A2 = W^T from the packed map, one 64 x 64 block per work-group through LDS.
__global__ __launch_bounds__(256) void k_unpack_transpose(PrepArgs pa, int64_t d) {
    const bf16_t* Wp = pa.W[blockIdx.z];
    bf16_t* A2 = pa.A2[blockIdx.z];
    __shared__ uint16_t tile[64][64 + 2];   // [o][i]
    const int64_t ib = blockIdx.x, ob = blockIdx.y;
    for (int c = threadIdx.x; c < 512; c += 256) {
        const int ol = c >> 3, ic = (c & 7) * 8;
        const u32x4 v = *(const u32x4*)(Wp + packed_index(ob * 64 + ol, (int)(ib * 64 + ic), d));
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            tile[ol][ic + 2 * k] = (uint16_t)(v[k] & 0xffffu);
            tile[ol][ic + 2 * k + 1] = (uint16_t)(v[k] >> 16);
        }
    }
    __syncthreads();
    for (int c = threadIdx.x; c < 512; c += 256) {
        const int il = c >> 3, oc = (c & 7) * 8;
        u32x4 v;
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = (uint32_t)tile[oc + 2 * k][il] | ((uint32_t)tile[oc + 2 * k + 1][il] << 16);
        *(u32x4*)(A2 + (ib * 64 + il) * d + ob * 64 + oc) = v;
    }
}

__device__ inline float bf16_to_f32(uint32_t bits16) { return __builtin_bit_cast(float, bits16 << 16); }

// One wave per packed row p of [W_k; W_v] (4 rows per work-group): B2[p] = [hi | lo] of the row
// scaled by gamma (the product rounded to fp32, then split into two bf16 parts), and the row's
// intercept c = sum_o W[p][o] gamma_o b_o (fp64: each lane's 8-column chunks in order, then a
// fixed shuffle tree) at its source row's index.
__global__ __launch_bounds__(256) void k_kv_split(PrepArgs pa, int64_t d, int kvw, int hd) {
    const int g = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int p = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (p >= 2 * kvw) return;
    const bf16_t *Wk = pa.Wk[g], *Wv = pa.Wv[g];
    const float *gamma = pa.gamma[g], *b = pa.b[g];
    bf16_t* B2 = pa.B2[g];
    float *ck = pa.ck[g], *cv = pa.cv[g];
    const bool is_k = p < kvw;
    const int pr = is_k ? p : p - kvw;
    const bf16_t* src = is_k ? Wk : Wv;
    bf16_t* row = B2 + (int64_t)p * 2 * d;
    double acc = 0.0;
    for (int64_t o = 8 * lane; o < d; o += 8 * 64) {
        const u32x4 v = *(const u32x4*)(src + packed_index(pr, (int)o, d));
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            float s[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const float w = bf16_to_f32(e == 0 ? (v[k] & 0xffffu) : (v[k] >> 16));
                s[e] = w * gamma[o + 2 * k + e];
                acc += (double)w * (double)gamma[o + 2 * k + e] * (double)b[o + 2 * k + e];
            }
            hi[k] = pack_bf16x2(s[0], s[1]);
            const float h0 = bf16_to_f32(hi[k] & 0xffffu), h1 = bf16_to_f32(hi[k] >> 16);
            lo[k] = pack_bf16x2(s[0] - h0, s[1] - h1);
        }
        *(u32x4*)(row + o) = u32x4{hi[0], hi[1], hi[2], hi[3]};
        *(u32x4*)(row + d + o) = u32x4{lo[0], lo[1], lo[2], lo[3]};
    }
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (lane == 0) {
        const int f = (pr / kCT) * kCT + packed_source_row(pr % kCT, hd);
        (is_k ? ck : cv)[f] = (float)acc;
    }
}

struct ComposeArgs {
    int64_t d;
    int32_t kvw;
    int32_t nf;            // d / 256
    int32_t n_t;           // tiles of T per layer: nf (nf + 1) / 2
    int32_t n_tiles;       // tiles per layer: n_t + nf * 2 kvw / 256
    const bf16_t* A2[kComposeGroup];   // [d][d] per layer: W^T
    const bf16_t* B2[kComposeGroup];   // [2 kvw][2d] per layer
    bf16_t* T[kComposeGroup];
    float* gdiag[kComposeGroup];       // q + d: the diagonal of W^T W
    bf16_t* Mk[kComposeGroup];
    bf16_t* Mv[kComposeGroup];
};

__global__ __launch_bounds__(PipeGemm::kThr) void k_compose_gemm(ComposeArgs a) {
    using G = PipeGemm;
    __shared__ __attribute__((aligned(16))) char lds[G::LDS_BYTES];
    const int u = xcd_order((int)blockIdx.x, (int)gridDim.x);
    const int l = u / a.n_tiles, v = u - l * a.n_tiles;
    const int64_t d = a.d;
    const bf16_t* A2 = a.A2[l];
    G gm;
    if (v < a.n_t) {
        // T tile (I, J), J >= I: acc[j][i] = (W^T W)[j][i]; rows j are A, rows i are B.
        // Row tiles I in groups of 4; within a group, columns J in order and the group's rows
        // with I <= J fastest, so the 32 tiles an XCD runs at once read about 4 + 8 strips of W
        // instead of 2 + 16
        int I = 0, J = 0, rem = v;
        for (int i0 = 0; i0 < a.nf; i0 += 4) {
            const int gs = a.nf - i0 < 4 ? a.nf - i0 : 4;
            int size = 0;
            for (int j = i0; j < a.nf; ++j) size += (j - i0 + 1) < gs ? (j - i0 + 1) : gs;
            if (rem < size) {
                for (J = i0;; ++J) {
                    const int c = (J - i0 + 1) < gs ? (J - i0 + 1) : gs;
                    if (rem < c) break;
                    rem -= c;
                }
                I = i0 + rem;
                break;
            }
            rem -= size;
        }
        gm.run(lds, PipeOperand{A2 + (int64_t)J * kCT * d, d, kCT}, PipeOperand{A2 + (int64_t)I * kCT * d, d, kCT},
               (int)(d / G::BK));
#pragma unroll
        for (int jb = 0; jb < G::SN; ++jb) {
            const int64_t i = (int64_t)I * kCT + G::col_of(jb);
#pragma unroll
            for (int ib = 0; ib < G::SM; ++ib)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int64_t j0 = (int64_t)J * kCT + G::row_of(ib, 4 * q);
                    float t[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int64_t j = j0 + e;
                        const float g = gm.acc[ib][jb][4 * q + e];
                        t[e] = j > i ? 2.f * g : 0.f;
                        if (j == i) a.gdiag[l][i] = g;   // kept in fp32: the quadratic form's heaviest terms
                    }
                    *(u32x2*)(a.T[l] + packed_index(i, (int)j0, d)) =
                        u32x2{pack_bf16x2(t[0], t[1]), pack_bf16x2(t[2], t[3])};
                }
        }
    } else {
        // M tile: acc[i][p] = sum_o W[o][i] (W_kv diag(gamma))[p][o] over K = 2d (hi, lo)
        // in groups of 4 row tiles F of W_kv, each against all d / 256 column tiles I of W
        int F, I;
        grouped_tile(v - a.n_t, 2 * a.kvw / kCT, a.nf, 4, F, I);
        // K = 2d: the hi and lo halves of B2 against the same W^T rows (A's k-steps fold back)
        gm.run(lds, PipeOperand{A2 + (int64_t)I * kCT * d, d, kCT},
               PipeOperand{a.B2[l] + (int64_t)F * kCT * 2 * d, 2 * d, kCT}, (int)(2 * d / G::BK), (int)(d / G::BK));
#pragma unroll
        for (int jb = 0; jb < G::SN; ++jb) {
            const int p = F * kCT + G::col_of(jb);
            bf16_t* dst = p < a.kvw ? a.Mk[l] : a.Mv[l];
            const int pr = p < a.kvw ? p : p - a.kvw;
#pragma unroll
            for (int ib = 0; ib < G::SM; ++ib)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int i0 = I * kCT + G::row_of(ib, 4 * q);
                    const f32x16& c = gm.acc[ib][jb];
                    *(u32x2*)(dst + packed_index(pr, i0, d)) =
                        u32x2{pack_bf16x2(c[4 * q], c[4 * q + 1]), pack_bf16x2(c[4 * q + 2], c[4 * q + 3])};
                }
        }
    }
}

// q[i] = 2 sum_o W[o][i] b[o] (one wave per i, reading row i of W^T), q[2d] = |b|^2 (the last
// work-group); fp64 sums in a fixed order.
__global__ __launch_bounds__(256) void k_qvec(PrepArgs pa, int64_t d) {
    const bf16_t* A2 = pa.A2[blockIdx.y];
    const float* b = pa.b[blockIdx.y];
    float* q = pa.q[blockIdx.y];
    __shared__ double red[256];
    if ((int64_t)blockIdx.x * 4 >= d) {
        double s = 0.0;
        for (int64_t o = threadIdx.x; o < d; o += 256) s += (double)b[o] * (double)b[o];
        red[threadIdx.x] = s;
        __syncthreads();
        for (int h = 128; h > 0; h >>= 1) {
            if ((int)threadIdx.x < h) red[threadIdx.x] += red[threadIdx.x + h];
            __syncthreads();
        }
        if (threadIdx.x == 0) q[2 * d] = (float)red[0];
        return;
    }
    const int lane = threadIdx.x & 63;
    const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const bf16_t* row = A2 + i * d;
    double s = 0.0;
    // 8 consecutive columns per lane and load
    for (int64_t o = 8 * lane; o < d; o += 8 * 64) {
        const u32x4 v = *(const u32x4*)(row + o);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            s += (double)bf16_to_f32(v[k] & 0xffffu) * (double)b[o + 2 * k];
            s += (double)bf16_to_f32(v[k] >> 16) * (double)b[o + 2 * k + 1];
        }
    }
    for (int off = 32; off > 0; off >>= 1) {
        const double t = __shfl_xor(s, off);
        s += t;
    }
    if (lane == 0) q[i] = (float)(2.0 * s);
}

// One layer slot of the workspace: A2, then B2.
static size_t compose_ws(int64_t d, int64_t kvw, size_t* off_b2) {
    const size_t a2 = round_up((size_t)d * d * 2, 256);
    if (off_b2) *off_b2 = a2;
    return a2 + round_up((size_t)2 * kvw * 2 * d * 2, 256);
}

}  // namespace rf

using namespace rf;

extern "C" {

size_t rf_fill_compose_workspace_bytes(const rf_fill_weights* w) {
    if (!w || w->d <= 0 || w->d % kCT != 0 || w->n_kv_heads <= 0 || w->head_dim <= 0) return 0;
    return compose_ws(w->d, (int64_t)w->n_kv_heads * w->head_dim, nullptr);
}

rf_status rf_fill_compose(const rf_fill_weights* w, int32_t n_layers, void* const* T, float* const* q,
                          void* const* M_k, void* const* M_v, float* const* c_k, float* const* c_v, void* d_ws,
                          size_t ws_bytes, void* stream) {
    clear_error();
    RF_REQUIRE(w, RF_ERR_INVALID_ARG, "rf_fill_compose: null weights");
    RF_REQUIRE(n_layers >= 0, RF_ERR_INVALID_ARG, "rf_fill_compose: n_layers must be >= 0");
    RF_REQUIRE(w->dtype == RF_BF16, RF_ERR_UNSUPPORTED, "rf_fill_compose: BF16 weights only");
    RF_REQUIRE(!w->map_scale, RF_ERR_UNSUPPORTED, "rf_fill_compose: int8 maps are not composed (use bf16 maps)");
    RF_REQUIRE(w->d > 0 && w->d % kCT == 0 && w->d <= (1 << 16), RF_ERR_UNSUPPORTED,
               "rf_fill_compose: d must be a positive multiple of 256, at most 65536");
    RF_REQUIRE(w->head_dim == 64 || w->head_dim == 128, RF_ERR_UNSUPPORTED, "rf_fill_compose: head_dim must be 64 or 128");
    const int64_t kvw = (int64_t)w->n_kv_heads * w->head_dim;
    RF_REQUIRE(w->n_kv_heads > 0 && kvw % kCT == 0, RF_ERR_UNSUPPORTED,
               "rf_fill_compose: n_kv_heads*head_dim must be a positive multiple of 256");
    if (n_layers == 0) return RF_OK;
    RF_REQUIRE(w->W_map && w->b_map && w->gamma && w->W_k && w->W_v && T && q && M_k && M_v && c_k && c_v && d_ws,
               RF_ERR_INVALID_ARG, "rf_fill_compose: null pointer argument");
    for (int l = 0; l < n_layers; ++l) {
        RF_REQUIRE(w->W_map[l] && w->b_map[l] && w->gamma[l] && w->W_k[l] && w->W_v[l] && T[l] && q[l] && M_k[l] &&
                       M_v[l] && c_k[l] && c_v[l],
                   RF_ERR_INVALID_ARG, "rf_fill_compose: null per-layer pointer");
        RF_REQUIRE(aligned(w->W_map[l], 16) && aligned(w->W_k[l], 16) && aligned(w->W_v[l], 16) && aligned(T[l], 16) &&
                       aligned(M_k[l], 16) && aligned(M_v[l], 16) && aligned(q[l], 16) && aligned(c_k[l], 16) &&
                       aligned(c_v[l], 16),
                   RF_ERR_INVALID_ARG, "rf_fill_compose: per-layer buffers must be 16-byte aligned");
    }
    size_t off_b2 = 0;
    const size_t slot = compose_ws(w->d, kvw, &off_b2);
    RF_REQUIRE(aligned(d_ws, 256), RF_ERR_INVALID_ARG, "rf_fill_compose: workspace must be 256-byte aligned");
    RF_REQUIRE(ws_bytes >= slot, RF_ERR_WORKSPACE, "rf_fill_compose: workspace too small");
    hipStream_t s = (hipStream_t)stream;
    const int64_t d = w->d;
    const int group = (int)std::min<size_t>({(size_t)n_layers, (size_t)kComposeGroup, ws_bytes / slot});
    ComposeArgs ca{};
    ca.d = d; ca.kvw = (int32_t)kvw; ca.nf = (int32_t)(d / kCT);
    ca.n_t = ca.nf * (ca.nf + 1) / 2;
    ca.n_tiles = ca.n_t + (int32_t)(ca.nf * (2 * kvw / kCT));
    for (int l0 = 0; l0 < n_layers; l0 += group) {
        const int gsz = std::min(group, n_layers - l0);
        PrepArgs pa{};
        for (int g = 0; g < gsz; ++g) {
            const int l = l0 + g;
            bf16_t* A2 = (bf16_t*)((char*)d_ws + (size_t)g * slot);
            bf16_t* B2 = (bf16_t*)((char*)A2 + off_b2);
            pa.W[g] = (const bf16_t*)w->W_map[l]; pa.Wk[g] = (const bf16_t*)w->W_k[l];
            pa.Wv[g] = (const bf16_t*)w->W_v[l]; pa.gamma[g] = w->gamma[l]; pa.b[g] = w->b_map[l];
            pa.A2[g] = A2; pa.B2[g] = B2; pa.ck[g] = c_k[l]; pa.cv[g] = c_v[l]; pa.q[g] = q[l];
            ca.A2[g] = A2; ca.B2[g] = B2;
            ca.T[g] = (bf16_t*)T[l]; ca.gdiag[g] = q[l] + d; ca.Mk[g] = (bf16_t*)M_k[l]; ca.Mv[g] = (bf16_t*)M_v[l];
        }
        // the layers' preparations, each one launch over the group
        hipLaunchKernelGGL(k_unpack_transpose, dim3((unsigned)(d / 64), (unsigned)(d / 64), (unsigned)gsz), dim3(256),
                           0, s, pa, d);
        RF_TRY_LAUNCH("rf_fill_compose: transpose");
        hipLaunchKernelGGL(k_kv_split, dim3((unsigned)ceil_div(2 * kvw, 4), (unsigned)gsz), dim3(256), 0, s, pa, d, (int)kvw,
                           w->head_dim);
        RF_TRY_LAUNCH("rf_fill_compose: scaled projections");
        hipLaunchKernelGGL(k_qvec, dim3((unsigned)(d / 4 + 1), (unsigned)gsz), dim3(256), 0, s, pa, d);
        RF_TRY_LAUNCH("rf_fill_compose: sum-of-squares vector");
        hipLaunchKernelGGL(k_compose_gemm, dim3((unsigned)(gsz * ca.n_tiles)), dim3(PipeGemm::kThr), 0, s, ca);
        RF_TRY_LAUNCH("rf_fill_compose: products");
    }
    return RF_OK;
}

}  // extern "C"
