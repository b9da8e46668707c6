// Gated DeltaNet state update over a token range (RidgeFill project page, "Method" step 3: on
// a Gated DeltaNet layer the filled rows also run the layer's state update).  Per layer and
// head, the published recurrence
//     S_t = exp(g_t) S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T      (S: d_v x d_k)
// with k_t optionally L2-normalised.  Row r of S evolves on its own:
//     s_r <- a s_r + c k,   c = beta (v_r - a (s_r . k)),   a = exp(g)
// (with normalised keys k -> k rn, rn = 1/sqrt(|k|^2 + eps): c = beta (v_r - a (s_r . k) rn) rn).
// Each row is held by d_k / 8 consecutive lanes (8 fp32 registers each; the row's dot product
// reduced over them by DPP lane moves, no LDS round trip), 256 / (d_k / 8) rows per
// work-group of 256 threads.  Tokens go in blocks of 32: a block's keys, values and gates are
// staged in LDS (keys as stored) while the next block's rows are in flight in registers,
// so the sequential token loop reads only LDS (a block's reads issued ahead of the chain);
// each block's key norms are computed once, 8 lanes per token, when it is staged.
// Within a block the state is carried scaled, u = s / A_t with A_t the product of the block's
// decays up to token t, so a token's update is u <- u + c' k (one fused multiply-add per
// element instead of a multiply and a fused multiply-add):
//     s_{t-1} . k = A_{t-1} (u . k),   c' = c / A_t = p_t (v_r - q_t (u . k)),
//     q_t = rn A_t,   p_t = beta rn / A_t,
// and s = A_31 u at the block's end.  This is the same recurrence regrouped (the rounding of
// the sum is relative to the same magnitudes after the final scaling); it is used for a block
// only when every A_t lies in [2^-60, 2^60], so that neither u nor 1 / A_t can overflow, and
// the block runs the direct form otherwise.
#include <math.h>

#include <string>

#include "rf_internal.h"
#include "rf_mfma.h"
#include "rf_pipe.h"

namespace rf {

constexpr int kGdnMaxLayers = 64;
constexpr int kGdnElems = 8;          // state elements per lane
constexpr int kGdnBlock = 32;         // tokens per staged block
// lanes per state row and rows per work-group for a key width
__host__ __device__ constexpr int gdn_lanes(int dk) { return dk / kGdnElems; }
__host__ __device__ constexpr int gdn_rows(int dk) { return 256 / gdn_lanes(dk); }

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

// Element i's stored bits, and their fp32 value (kept apart so that a prefetch holds the raw
// bits and converts them only where they are staged).
template <typename T> __device__ inline uint32_t ld_bits(const T* p, int64_t i);
template <> __device__ inline uint32_t ld_bits<float>(const float* p, int64_t i) {
    return __builtin_bit_cast(uint32_t, p[i]);
}
template <> __device__ inline uint32_t ld_bits<bf16_t>(const bf16_t* p, int64_t i) { return (uint32_t)p[i]; }
template <typename T> __device__ inline float bits_f32(uint32_t b) {
    return sizeof(T) == 2 ? __builtin_bit_cast(float, b << 16) : __builtin_bit_cast(float, b);
}

// A DPP lane move within each row of 16 lanes (dpp_ctrl CTRL), every lane a source.
template <int CTRL>
__device__ inline float dpp_move(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
// The sum over each group of LANES (8 or 16) consecutive lanes, in every lane of the group:
// lane ^ 1, lane ^ 2 (quad permutes), then the mirrored lane of the other quad (half-row
// mirror) and, for 16, of the other half-row (row mirror).  A fixed order.
template <int LANES>
__device__ inline float group_sum(float x) {
    x += dpp_move<0xB1>(x);     // quad_perm [1, 0, 3, 2]
    x += dpp_move<0x4E>(x);     // quad_perm [2, 3, 0, 1]
    x += dpp_move<0x141>(x);    // row_half_mirror
    if constexpr (LANES == 16) x += dpp_move<0x140>(x);   // row_mirror
    return x;
}

template <typename T, int DK>
__device__ inline void gdn_state(const GdnArgs& a) {
    constexpr int E = kGdnElems, LANES = gdn_lanes(DK), ROWS = gdn_rows(DK);
    static_assert(LANES == 8 || LANES == 16, "8 or 16 lanes per state row");
    // the staged block: keys [32][DK] (fp32), values [32][ROWS rows of this work-group], gate a,
    // beta, key norm factor.  One buffer: the next block waits in registers until every lane is
    // done with this one.
    __shared__ __attribute__((aligned(16))) float sk[kGdnBlock][DK];
    __shared__ float sv[kGdnBlock][ROWS];
    __shared__ float sa[kGdnBlock], sb[kGdnBlock], sn[kGdnBlock], sg[kGdnBlock];
    __shared__ __attribute__((aligned(16))) float sqp[kGdnBlock][2];   // scaled form: q_t, p_t
    __shared__ __attribute__((aligned(16))) int32_t sok[kGdnBlock];     // A_t in range
    __shared__ float sA;                                                // A_31
    const int per_layer = a.n_heads * a.wg_per_head;
    // the work-groups of one head on one XCD, so the head's key rows, which every one of them
    // reads, come from that XCD's L2 after the first
    const int bid = xcd_order((int)blockIdx.x, (int)gridDim.x);
    const int l = bid / per_layer;
    const int rem = bid - l * per_layer;
    const int h = rem / a.wg_per_head;
    const int r0 = (rem - h * a.wg_per_head) * ROWS;
    const int t = threadIdx.x;
    const int rl = t / LANES;                    // this lane's state row within the work-group
    const int row = r0 + rl;
    const int j0 = (t % LANES) * E;              // and its columns
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
    constexpr int KVEC = 16 / (int)sizeof(T);                 // key elements per 16-byte load
    constexpr int KPER = kGdnBlock * DK / (256 * KVEC);       // key loads per thread per block
    constexpr int VPER = kGdnBlock * ROWS / 256;
    // Every load is issued unconditionally at an in-range index (tokens past the range read the
    // last token, rows past d_v the last row) and masked when staged: a load guarded by a
    // branch would be waited for on the spot instead of under the next block's token loop.
    u32x4 rk[KPER];
    uint32_t rv[VPER];
    float rg = 0.f, rb = 0.f;
    auto fetch = [&](int64_t tb) {
#pragma unroll
        for (int i = 0; i < KPER; ++i) {
            const int e = (t + 256 * i) * KVEC, tt = e / DK, jj = e % DK;
            const int64_t tok = tb + tt < a.T ? tb + tt : a.T - 1;
            rk[i] = *(const u32x4*)(K + tok * a.ld_k + jj);
        }
#pragma unroll
        for (int i = 0; i < VPER; ++i) {
            const int e = t + 256 * i, tt = e / ROWS, rr = e % ROWS;
            const int64_t tok = tb + tt < a.T ? tb + tt : a.T - 1;
            const int r = r0 + rr < a.d_v ? r0 + rr : a.d_v - 1;
            rv[i] = ld_bits<T>(V, tok * a.ld_v + r);
        }
        if (t < kGdnBlock) {
            const int64_t tok = tb + t < a.T ? tb + t : a.T - 1;
            rg = G[tok * a.n_heads];
            rb = B[tok * a.n_heads];
        }
    };
    auto stage = [&](int64_t tb) {
#pragma unroll
        for (int i = 0; i < KPER; ++i) {
            const int e = (t + 256 * i) * KVEC;
            const u32x4 v = tb + e / DK < a.T ? rk[i] : u32x4{0u, 0u, 0u, 0u};
            float* dst = &sk[e / DK][e % DK];
            if constexpr (sizeof(T) == 2) {
                *(f32x4*)dst = f32x4{__builtin_bit_cast(float, v[0] << 16), __builtin_bit_cast(float, v[0] & 0xffff0000u),
                                     __builtin_bit_cast(float, v[1] << 16), __builtin_bit_cast(float, v[1] & 0xffff0000u)};
                *(f32x4*)(dst + 4) =
                    f32x4{__builtin_bit_cast(float, v[2] << 16), __builtin_bit_cast(float, v[2] & 0xffff0000u),
                          __builtin_bit_cast(float, v[3] << 16), __builtin_bit_cast(float, v[3] & 0xffff0000u)};
            } else {
                *(u32x4*)dst = v;
            }
        }
#pragma unroll
        for (int i = 0; i < VPER; ++i) {
            const int e = t + 256 * i;
            sv[e / ROWS][e % ROWS] = tb + e / ROWS < a.T ? bits_f32<T>(rv[i]) : 0.f;
        }
        if (t < kGdnBlock) {
            const bool ok = tb + t < a.T;
            sa[t] = ok ? expf(rg) : 1.f;
            sb[t] = ok ? rb : 0.f;
            sg[t] = ok ? rg : 0.f;
        }
    };
    // key norm factors of a staged block: 8 lanes per token, each summing DK / 8 squares, then
    // over the 8 lanes; 1 / sqrt(|k|^2 + eps), 1 without normalisation, 0 past the range
    auto norms = [&](int64_t tb) {
        constexpr int PART = DK / 8;
        const int tt = t / 8, p0 = (t % 8) * PART;
        float q = 0.f;
#pragma unroll
        for (int c = 0; c < PART; c += 4) {
            const f32x4 v = *(const f32x4*)&sk[tt][p0 + c];
            q += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
        }
        q = group_sum<8>(q);
        if (t % 8 == 0) {
            const float rn = tb + tt >= a.T ? 0.f : (a.normalise ? 1.0f / sqrtf(q + a.eps) : 1.0f);
            sn[tt] = rn;
            // the scaled form's factors: the block's log-decay up to this token, summed in
            // token order (the same order in every thread that needs it)
            float G = 0.f;
            for (int i = 0; i <= tt; ++i) G += sg[i];
            const float At = expf(G);
            sok[tt] = G >= -41.0f && G <= 41.0f;   // |G| <= 60 ln 2
            sqp[tt][0] = rn * At;
            sqp[tt][1] = sb[tt] * rn / At;
            if (tt == kGdnBlock - 1) sA = At;
        }
    };
    const int n_blocks = (int)((a.T + kGdnBlock - 1) / kGdnBlock);
    fetch(0);
    stage(0);
    __syncthreads();
    norms(0);
    __syncthreads();
    for (int blk = 0; blk < n_blocks; ++blk) {
        const int64_t tb = (int64_t)blk * kGdnBlock;
        if (blk + 1 < n_blocks) fetch(tb + kGdnBlock);
        // a fixed trip count, unrolled, so each token's LDS reads are issued ahead of the chain.
        // Tokens past the range were staged as zero keys and values with gate 1, strength 0
        // and norm factor 0: their update is exactly s <- s.
        // the block's form, the same in every thread (all read the same flags)
        bool scaled = true;
#pragma unroll
        for (int i = 0; i < kGdnBlock; i += 4) {
            const int4 f = *(const int4*)&sok[i];
            scaled = scaled && f.x && f.y && f.z && f.w;
        }
        if (scaled) {
#pragma unroll 4
            for (int tt = 0; tt < kGdnBlock; ++tt) {
                const f32x4 k0 = *(const f32x4*)&sk[tt][j0], k1 = *(const f32x4*)&sk[tt][j0 + 4];
                const float k[E] = {k0[0], k0[1], k0[2], k0[3], k1[0], k1[1], k1[2], k1[3]};
                const float qv = sqp[tt][0], pv = sqp[tt][1], vr = sv[tt][rl];
                float d0 = s[0] * k[0], d1 = s[1] * k[1];
#pragma unroll
                for (int e = 2; e < E; e += 2) {
                    d0 += s[e] * k[e];
                    d1 += s[e + 1] * k[e + 1];
                }
                const float dot = group_sum<LANES>(d0 + d1);
                const float c = pv * (vr - qv * dot);
#pragma unroll
                for (int e = 0; e < E; ++e) s[e] += c * k[e];
            }
            const float Ab = sA;
#pragma unroll
            for (int e = 0; e < E; ++e) s[e] *= Ab;
        } else {
#pragma unroll 4
            for (int tt = 0; tt < kGdnBlock; ++tt) {
                const f32x4 k0 = *(const f32x4*)&sk[tt][j0], k1 = *(const f32x4*)&sk[tt][j0 + 4];
                const float k[E] = {k0[0], k0[1], k0[2], k0[3], k1[0], k1[1], k1[2], k1[3]};
                const float av = sa[tt], bv = sb[tt], rn = sn[tt], vr = sv[tt][rl];
                // the row's dot product: two partial sums, then over the row's lanes
                float d0 = s[0] * k[0], d1 = s[1] * k[1];
#pragma unroll
                for (int e = 2; e < E; e += 2) {
                    d0 += s[e] * k[e];
                    d1 += s[e + 1] * k[e + 1];
                }
                const float dot = group_sum<LANES>(d0 + d1);
                const float c = bv * (vr - av * dot * rn) * rn;
#pragma unroll
                for (int e = 0; e < E; ++e) s[e] = av * s[e] + c * k[e];
            }
        }
        __syncthreads();   // every lane is done with this block's buffer
        if (blk + 1 < n_blocks) {
            stage(tb + kGdnBlock);
            __syncthreads();
            norms(tb + kGdnBlock);
            __syncthreads();
        }
    }
    if (live) {
#pragma unroll
        for (int e = 0; e < E; ++e) S[e] = s[e];
    }
}

// Six waves per SIMD for bf16 keys (at most 85 registers): 16-row work-groups of a 16-head set
// of layers are then resident at once, not in one and a half rounds.
template <int DK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(6))) void k_gdn_state_bf16(GdnArgs a) {
    gdn_state<bf16_t, DK>(a);
}
template <int DK>
__global__ __launch_bounds__(256) void k_gdn_state_f32(GdnArgs a) {
    gdn_state<float, DK>(a);
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
    RF_REQUIRE(ld_k * (int64_t)elem_bytes(desc->dtype) % 16 == 0, RF_ERR_INVALID_ARG,
               "rf_gdn_state: the key row stride must be a multiple of 16 bytes");
    if (n_layers == 0 || n_tokens == 0) return RF_OK;
    RF_REQUIRE(d_k && d_v && d_g && d_beta && d_state, RF_ERR_INVALID_ARG, "rf_gdn_state: null pointer argument");
    for (int l = 0; l < n_layers; ++l) {
        RF_REQUIRE(d_k[l] && d_v[l] && d_g[l] && d_beta[l] && d_state[l], RF_ERR_INVALID_ARG,
                   "rf_gdn_state: null per-layer pointer");
        RF_REQUIRE(aligned(d_state[l], 16) && aligned(d_k[l], 16), RF_ERR_INVALID_ARG,
                   "rf_gdn_state: states and key rows must be 16-byte aligned");
    }
    GdnArgs a{};
    a.n_heads = desc->n_heads; a.d_v = desc->d_v; a.wg_per_head = (int32_t)ceil_div(desc->d_v, gdn_rows(desc->d_k));
    a.T = n_tokens; a.ld_k = ld_k; a.ld_v = ld_v; a.normalise = desc->normalise_k; a.eps = desc->eps;
    for (int l = 0; l < n_layers; ++l) {
        a.k[l] = d_k[l]; a.v[l] = d_v[l]; a.g[l] = d_g[l]; a.beta[l] = d_beta[l]; a.S[l] = d_state[l];
    }
    const dim3 grid((unsigned)(n_layers * desc->n_heads * a.wg_per_head));
    hipStream_t s = (hipStream_t)stream;
    if (desc->dtype == RF_BF16) {
        if (desc->d_k == 128) hipLaunchKernelGGL((k_gdn_state_bf16<128>), grid, dim3(256), 0, s, a);
        else hipLaunchKernelGGL((k_gdn_state_bf16<64>), grid, dim3(256), 0, s, a);
    } else {
        if (desc->d_k == 128) hipLaunchKernelGGL((k_gdn_state_f32<128>), grid, dim3(256), 0, s, a);
        else hipLaunchKernelGGL((k_gdn_state_f32<64>), grid, dim3(256), 0, s, a);
    }
    return check_launch("rf_gdn_state");
}

}  // extern "C"
