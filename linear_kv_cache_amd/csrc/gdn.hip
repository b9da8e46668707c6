// Gated DeltaNet state update over a token range (RidgeFill project page, "Method" step 3: on
// a Gated DeltaNet layer the filled rows also run the layer's state update).  Per layer and
// head, the published recurrence
//     S_t = exp(g_t) S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T      (S: d_v x d_k)
// with k_t optionally L2-normalised.  Row r of S evolves on its own:
//     s_r <- a s_r + c k,   c = beta (v_r - a (s_r . k)),   a = exp(g)
// (with normalised keys k -> k rn, rn = 1/sqrt(|k|^2 + eps): c = beta (v_r - a (s_r . k) rn) rn).
// Each row is held by 8 consecutive lanes (d_k / 8 fp32 registers each, the row's dot product
// reduced over them by lane exchanges), 32 rows per work-group of 256 threads.  Tokens go in
// blocks of 32: a block's keys, values, gates and key norms are staged in LDS (fp32) while the
// next block's rows are in flight in registers, so the sequential token loop reads only LDS.
#include <math.h>

#include <string>

#include "rf_internal.h"
#include "rf_mfma.h"

namespace rf {

constexpr int kGdnMaxLayers = 64;
constexpr int kGdnLanes = 8;          // lanes per state row
constexpr int kGdnRows = 256 / kGdnLanes;   // rows per work-group
constexpr int kGdnBlock = 32;         // tokens per staged block

struct GdnArgs {
    int32_t n_heads, d_v, wg_per_head;
    int64_t T, ld_k, ld_v;
    int32_t normalise;
    float eps;
    const void* k[kGdnMaxLayers];
    const void* v[kGdnMaxLayers];
    const float* g[kGdnMaxLayers];
    const float* beta[kGdnMaxLayers];
    float* S[kGdnMaxLayers];
};

template <typename T> __device__ inline float ld_elem(const T* p, int64_t i);
template <> __device__ inline float ld_elem<float>(const float* p, int64_t i) { return p[i]; }
template <> __device__ inline float ld_elem<bf16_t>(const bf16_t* p, int64_t i) {
    return __builtin_bit_cast(float, (uint32_t)p[i] << 16);
}

template <typename T, int DK>
__global__ __launch_bounds__(256) void k_gdn_state(GdnArgs a) {
    constexpr int E = DK / kGdnLanes;   // state elements per lane
    // per block: keys [32][DK], values [32][32 rows of this work-group], gate a, beta, 1/|k|
    __shared__ float sk[2][kGdnBlock][DK];
    __shared__ float sv[2][kGdnBlock][kGdnRows];
    __shared__ float sa[2][kGdnBlock], sb[2][kGdnBlock], sn[2][kGdnBlock];
    const int per_layer = a.n_heads * a.wg_per_head;
    const int l = blockIdx.x / per_layer;
    const int rem = blockIdx.x - l * per_layer;
    const int h = rem / a.wg_per_head;
    const int r0 = (rem - h * a.wg_per_head) * kGdnRows;
    const int t = threadIdx.x;
    const int row = r0 + t / kGdnLanes;          // this lane's state row
    const int j0 = (t % kGdnLanes) * E;          // and its columns
    const bool live = row < a.d_v;
    const T* K = (const T*)a.k[l] + (int64_t)h * DK;
    const T* V = (const T*)a.v[l] + (int64_t)h * a.d_v;
    const float* G = a.g[l] + h;
    const float* B = a.beta[l] + h;
    float* S = a.S[l] + ((int64_t)h * a.d_v + (live ? row : 0)) * DK + j0;
    float s[E];
#pragma unroll
    for (int e = 0; e < E; ++e) s[e] = live ? S[e] : 0.f;

    // staging: key elements of the block (32 * DK), one value per (token, row), per-token scalars
    constexpr int KPER = kGdnBlock * DK / 256;
    float rk[KPER], rv[kGdnBlock * kGdnRows / 256], rg = 0.f, rb = 0.f;
    auto fetch = [&](int64_t tb) {
#pragma unroll
        for (int i = 0; i < KPER; ++i) {
            const int e = t + 256 * i, tt = e / DK, jj = e % DK;
            rk[i] = tb + tt < a.T ? ld_elem<T>(K, (tb + tt) * a.ld_k + jj) : 0.f;
        }
#pragma unroll
        for (int i = 0; i < kGdnBlock * kGdnRows / 256; ++i) {
            const int e = t + 256 * i, tt = e / kGdnRows, rr = e % kGdnRows;
            rv[i] = (tb + tt < a.T && r0 + rr < a.d_v) ? ld_elem<T>(V, (tb + tt) * a.ld_v + r0 + rr) : 0.f;
        }
        if (t < kGdnBlock) {
            const bool ok = tb + t < a.T;
            rg = ok ? G[(tb + t) * a.n_heads] : 0.f;
            rb = ok ? B[(tb + t) * a.n_heads] : 0.f;
        }
    };
    auto stage = [&](int buf) {
#pragma unroll
        for (int i = 0; i < KPER; ++i) {
            const int e = t + 256 * i;
            sk[buf][e / DK][e % DK] = rk[i];
        }
#pragma unroll
        for (int i = 0; i < kGdnBlock * kGdnRows / 256; ++i) {
            const int e = t + 256 * i;
            sv[buf][e / kGdnRows][e % kGdnRows] = rv[i];
        }
        if (t < kGdnBlock) {
            sa[buf][t] = expf(rg);
            sb[buf][t] = rb;
        }
    };
    const int n_blocks = (int)((a.T + kGdnBlock - 1) / kGdnBlock);
    fetch(0);
    stage(0);
    __syncthreads();
    for (int blk = 0; blk < n_blocks; ++blk) {
        const int buf = blk & 1;
        const int64_t tb = (int64_t)blk * kGdnBlock;
        if (blk + 1 < n_blocks) fetch(tb + kGdnBlock);
        // the block's key norms (a wave's lane per token; the other lanes idle here)
        if (t < kGdnBlock) {
            float q = 0.f;
            if (a.normalise) {
#pragma unroll 8
                for (int jj = 0; jj < DK; ++jj) q += sk[buf][t][jj] * sk[buf][t][jj];
                sn[buf][t] = 1.0f / sqrtf(q + a.eps);
            } else {
                sn[buf][t] = 1.0f;
            }
        }
        __syncthreads();
        const int nt = (int)((a.T - tb) < kGdnBlock ? (a.T - tb) : kGdnBlock);
        for (int tt = 0; tt < nt; ++tt) {
            float k[E];
#pragma unroll
            for (int e = 0; e < E; e += 4) {
                const f32x4 q4 = *(const f32x4*)&sk[buf][tt][j0 + e];
                k[e] = q4[0]; k[e + 1] = q4[1]; k[e + 2] = q4[2]; k[e + 3] = q4[3];
            }
            float dot = 0.f;
#pragma unroll
            for (int e = 0; e < E; ++e) dot += s[e] * k[e];
            // the row's dot product over its 8 lanes (fixed order: xor 1, 2, 4)
            dot += __shfl_xor(dot, 1);
            dot += __shfl_xor(dot, 2);
            dot += __shfl_xor(dot, 4);
            const float av = sa[buf][tt], bv = sb[buf][tt], rn = sn[buf][tt];
            const float vr = sv[buf][tt][t / kGdnLanes];
            const float c = bv * (vr - av * dot * rn) * rn;
#pragma unroll
            for (int e = 0; e < E; ++e) s[e] = av * s[e] + c * k[e];
        }
        __syncthreads();   // every lane is done with this block's buffer
        if (blk + 1 < n_blocks) {
            stage(buf ^ 1);
            __syncthreads();
        }
    }
    if (live) {
#pragma unroll
        for (int e = 0; e < E; ++e) S[e] = s[e];
    }
}

}  // namespace rf

using namespace rf;

extern "C" {

rf_status rf_gdn_state(const rf_gdn_desc* desc, int32_t n_layers, const void* const* d_k, const void* const* d_v,
                       int64_t ld_k, int64_t ld_v, const float* const* d_g, const float* const* d_beta,
                       int64_t n_tokens, float* const* d_state, void* stream) {
    clear_error();
    RF_REQUIRE(desc, RF_ERR_INVALID_ARG, "rf_gdn_state: null descriptor");
    RF_REQUIRE(n_layers >= 0 && n_tokens >= 0, RF_ERR_INVALID_ARG, "rf_gdn_state: n_layers and n_tokens must be >= 0");
    RF_REQUIRE(n_layers <= kGdnMaxLayers, RF_ERR_UNSUPPORTED, "rf_gdn_state: at most 64 layers per call");
    RF_REQUIRE(valid_dtype(desc->dtype), RF_ERR_INVALID_ARG, "rf_gdn_state: bad dtype");
    RF_REQUIRE(desc->d_k == 64 || desc->d_k == 128, RF_ERR_UNSUPPORTED, "rf_gdn_state: d_k must be 64 or 128");
    RF_REQUIRE(desc->n_heads > 0 && desc->d_v > 0 && desc->d_v <= 4096, RF_ERR_INVALID_ARG,
               "rf_gdn_state: n_heads must be > 0 and d_v in [1, 4096]");
    RF_REQUIRE(desc->normalise_k == 0 || desc->normalise_k == 1, RF_ERR_INVALID_ARG,
               "rf_gdn_state: normalise_k must be 0 or 1");
    RF_REQUIRE(desc->eps >= 0.f && isfinite(desc->eps), RF_ERR_INVALID_ARG, "rf_gdn_state: eps must be finite and >= 0");
    RF_REQUIRE(ld_k >= (int64_t)desc->n_heads * desc->d_k && ld_v >= (int64_t)desc->n_heads * desc->d_v,
               RF_ERR_INVALID_ARG, "rf_gdn_state: key and value rows shorter than n_heads * d_k (d_v)");
    if (n_layers == 0 || n_tokens == 0) return RF_OK;
    RF_REQUIRE(d_k && d_v && d_g && d_beta && d_state, RF_ERR_INVALID_ARG, "rf_gdn_state: null pointer argument");
    for (int l = 0; l < n_layers; ++l) {
        RF_REQUIRE(d_k[l] && d_v[l] && d_g[l] && d_beta[l] && d_state[l], RF_ERR_INVALID_ARG,
                   "rf_gdn_state: null per-layer pointer");
        RF_REQUIRE(aligned(d_state[l], 16), RF_ERR_INVALID_ARG, "rf_gdn_state: states must be 16-byte aligned");
    }
    GdnArgs a{};
    a.n_heads = desc->n_heads; a.d_v = desc->d_v; a.wg_per_head = (int32_t)ceil_div(desc->d_v, kGdnRows);
    a.T = n_tokens; a.ld_k = ld_k; a.ld_v = ld_v; a.normalise = desc->normalise_k; a.eps = desc->eps;
    for (int l = 0; l < n_layers; ++l) {
        a.k[l] = d_k[l]; a.v[l] = d_v[l]; a.g[l] = d_g[l]; a.beta[l] = d_beta[l]; a.S[l] = d_state[l];
    }
    const dim3 grid((unsigned)(n_layers * desc->n_heads * a.wg_per_head));
    hipStream_t s = (hipStream_t)stream;
    if (desc->dtype == RF_BF16) {
        if (desc->d_k == 128) hipLaunchKernelGGL((k_gdn_state<bf16_t, 128>), grid, dim3(256), 0, s, a);
        else hipLaunchKernelGGL((k_gdn_state<bf16_t, 64>), grid, dim3(256), 0, s, a);
    } else {
        if (desc->d_k == 128) hipLaunchKernelGGL((k_gdn_state<float, 128>), grid, dim3(256), 0, s, a);
        else hipLaunchKernelGGL((k_gdn_state<float, 64>), grid, dim3(256), 0, s, a);
    }
    return check_launch("rf_gdn_state");
}

}  // extern "C"
