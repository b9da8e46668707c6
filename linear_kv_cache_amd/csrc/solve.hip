// Closed-form ridge solve from the one-pass statistics (RidgeFill project page, "Method"
// step 2: a ridge regression fitted once in closed form; intercept by mean-centring).
//
//   C  = S_xx - s_x^T s_x / n  (+ lambda I)        fp64, symmetric from the upper triangle
//   B  = S_yx,l - s_y,l^T s_x / n                  fp64, one row per (target, output)
//   C = L L^T                                      blocked right-looking Cholesky, 64-wide panels
//   C^-1 = L^-T L^-1                               blocked triangular solves on the identity
//   W  = B C^-1,  b = s_y/n - W (s_x/n)            one GEMM, then a row-wise dot
// Diagonal 64 x 64 blocks are factored and inverted inside one workgroup each; everything
// else is a tiled fp64 GEMM.  All reductions run in a fixed order.
#include <math.h>

#include "rf_internal.h"
#include "rf_mfma.h"

namespace rf {

constexpr int kNB = 64;        // Cholesky / triangular-solve block
constexpr int kMaxSel = 64;

// ---- tiled fp64 GEMM:  C = alpha * A * op(B) + beta * C -------------------------------------
// A [M][K] (lda); op(B) = B^T with B [N][K] (BT) or B [K][N] (!BT); beta == 0 never reads C.
template <bool BT>
__global__ __launch_bounds__(256) void k_dgemm(int64_t M, int64_t N, int64_t K, double alpha, const double* A,
                                               int64_t lda, const double* B, int64_t ldb, double beta, double* C,
                                               int64_t ldc) {
    constexpr int BM = 64, BN = 64, BK = 16;
    __shared__ double As[BK][BM + 1];
    __shared__ double Bs[BK][BN + 1];
    const int t = threadIdx.x;
    const int tx = t & 15, ty = t >> 4;
    const int64_t m0 = (int64_t)blockIdx.x * BM, n0 = (int64_t)blockIdx.y * BN;
    double acc[4][4] = {};
    for (int64_t k0 = 0; k0 < K; k0 += BK) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int idx = t + 256 * e;
            const int m = idx >> 4, k = idx & 15;
            const int64_t gm = m0 + m, gk = k0 + k;
            As[k][m] = (gm < M && gk < K) ? A[gm * lda + gk] : 0.0;
            if (BT) {
                const int64_t gn = n0 + m;
                Bs[k][m] = (gn < N && gk < K) ? B[gn * ldb + gk] : 0.0;
            } else {
                const int kk = idx >> 6, n = idx & 63;
                const int64_t gk2 = k0 + kk, gn = n0 + n;
                Bs[kk][n] = (gn < N && gk2 < K) ? B[gk2 * ldb + gn] : 0.0;
            }
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < BK; ++k) {
            double a[4], b[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) a[r] = As[k][ty + 16 * r];
#pragma unroll
            for (int c = 0; c < 4; ++c) b[c] = Bs[k][tx + 16 * c];
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int c = 0; c < 4; ++c) acc[r][c] = fma(a[r], b[c], acc[r][c]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int64_t gm = m0 + ty + 16 * r;
        if (gm >= M) continue;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int64_t gn = n0 + tx + 16 * c;
            if (gn >= N) continue;
            double v = alpha * acc[r][c];
            if (beta != 0.0) v += beta * C[gm * ldc + gn];
            C[gm * ldc + gn] = v;
        }
    }
}

__global__ void k_copy2d(const double* src, int64_t lds, double* dst, int64_t ldd, int64_t rows, int64_t cols) {
    const int64_t n = rows * cols;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = i / cols, c = i % cols;
        dst[r * ldd + c] = src[r * lds + c];
    }
}

__global__ void k_identity(double* R, int64_t d) {
    const int64_t n = d * d;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        R[i] = (i / d == i % d) ? 1.0 : 0.0;
}

__global__ void k_zero_int(int32_t* p) { *p = 0; }

// C[i][j] = S_xx[min(i,j)][max(i,j)] - s_x[i] s_x[j] / n
__global__ void k_centre_gram(const float* Sxx, const double* sx, const int64_t* np, int64_t d, double* C) {
    const double inv_n = 1.0 / (double)*np;
    const int64_t n = d * d;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n; idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t i = idx / d, j = idx % d;
        const int64_t lo = i < j ? i : j, hi = i < j ? j : i;
        C[idx] = (double)Sxx[lo * d + hi] - sx[i] * sx[j] * inv_n;
    }
}

// Adds lambda (absolute, or times the mean diagonal) to the diagonal; one workgroup.
__global__ __launch_bounds__(256) void k_add_lambda(double* C, int64_t d, double lambda, int rel) {
    __shared__ double red[256];
    double lam = lambda;
    if (rel) {
        double s = 0.0;
        for (int64_t i = threadIdx.x; i < d; i += 256) s += C[i * d + i];
        red[threadIdx.x] = s;
        __syncthreads();
        for (int w = 128; w > 0; w >>= 1) {
            if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
            __syncthreads();
        }
        lam = lambda * red[0] / (double)d;
    }
    for (int64_t i = threadIdx.x; i < d; i += 256) C[i * d + i] += lam;
}

struct CrossArgs {
    const float* Syx;
    const double* sy;
    const double* sx;
    const int64_t* np;
    int64_t d;
    int64_t rows;          // n_sel * d
    double* R;             // [rows][d]
    double* mu_y;          // [rows]
    int32_t tsel[kMaxSel];
};

__global__ void k_centre_cross(CrossArgs a) {
    const double inv_n = 1.0 / (double)*a.np;
    const int64_t n = a.rows * a.d;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n; idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t c = idx / a.d, i = idx % a.d;
        const int64_t s = c / a.d, o = c % a.d;
        const int64_t srow = (int64_t)a.tsel[s] * a.d + o;
        const double syv = a.sy[srow];
        a.R[idx] = (double)a.Syx[srow * a.d + i] - syv * a.sx[i] * inv_n;
        if (i == 0) a.mu_y[c] = syv * inv_n;
    }
}

// Factor the diagonal block J (already updated by all earlier panels) in place into L_JJ and
// write L_JJ^-1 into Dinv.  info receives the 1-based index of the first non-positive pivot.
__global__ __launch_bounds__(256) void k_chol_diag(double* C, int64_t d, int J, double* Dinv, int32_t* info) {
    __shared__ double a[kNB][kNB + 1];
    __shared__ double b[kNB][kNB + 1];
    const int t = threadIdx.x;
    const int64_t off = (int64_t)J * kNB;
    for (int idx = t; idx < kNB * kNB; idx += 256) {
        const int i = idx / kNB, k = idx % kNB;
        a[i][k] = C[(off + i) * d + off + k];
    }
    __syncthreads();
    for (int j = 0; j < kNB; ++j) {
        if (t == 0) {
            const double p = a[j][j];
            if (!(p > 0.0) && *info == 0) *info = (int32_t)(off + j + 1);
            a[j][j] = sqrt(p);
        }
        __syncthreads();
        for (int i = j + 1 + t; i < kNB; i += 256) a[i][j] /= a[j][j];
        __syncthreads();
        for (int idx = t; idx < kNB * kNB; idx += 256) {
            const int i = idx / kNB, k = idx % kNB;
            if (k > j && i >= k) a[i][k] -= a[i][j] * a[k][j];
        }
        __syncthreads();
    }
    // inverse of the lower triangle, one column per thread
    if (t < kNB) {
        const int c = t;
        for (int i = 0; i < kNB; ++i) {
            if (i < c) {
                b[i][c] = 0.0;
            } else if (i == c) {
                b[i][c] = 1.0 / a[c][c];
            } else {
                double s = 0.0;
                for (int k = c; k < i; ++k) s += a[i][k] * b[k][c];
                b[i][c] = -s / a[i][i];
            }
        }
    }
    __syncthreads();
    double* D = Dinv + (int64_t)J * kNB * kNB;
    for (int idx = t; idx < kNB * kNB; idx += 256) {
        const int i = idx / kNB, k = idx % kNB;
        C[(off + i) * d + off + k] = k <= i ? a[i][k] : 0.0;
        D[idx] = b[i][k];
    }
}

// b[c] = mu_y[c] - sum_i W[c][i] s_x[i] / n ; one wave per row.
__global__ __launch_bounds__(256) void k_bias(const double* W, const double* sx, const int64_t* np, const double* mu_y,
                                              int64_t d, int64_t rows, float* b) {
    const int64_t c = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (c >= rows) return;
    const double inv_n = 1.0 / (double)*np;
    double s = 0.0;
    for (int64_t i = lane; i < d; i += 64) s += W[c * d + i] * sx[i];
    for (int w = 32; w > 0; w >>= 1) s += __shfl_xor(s, w);
    if (lane == 0) b[c] = (float)(mu_y[c] - s * inv_n);
}

__global__ void k_store_w(const double* W, int64_t n, float* Wf, bf16_t* Wlp) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const double v = W[i];
        if (Wf) Wf[i] = (float)v;
        if (Wlp) Wlp[i] = __builtin_bit_cast(uint16_t, (__bf16)(float)v);
    }
}

// -------------------------------------------------------------------------------------------
struct SolveWs {
    double *C, *Cinv, *R, *W, *P, *Dinv, *mu_y;
    size_t total;
};

static SolveWs solve_ws(void* base, int64_t d, int64_t n_sel) {
    SolveWs w{};
    size_t off = 0;
    char* p = (char*)base;
    auto take = [&](size_t bytes) {
        double* r = (double*)(p ? p + off : nullptr);
        off += round_up(bytes, 256);
        return r;
    };
    const int64_t rows = n_sel * d;
    w.C = take(d * d * 8);
    w.Cinv = take(d * d * 8);
    w.R = take(rows * d * 8);
    w.W = take(rows * d * 8);
    w.P = take(d * kNB * 8);
    w.Dinv = take(d * kNB * 8);
    w.mu_y = take(rows * 8);
    w.total = off;
    return w;
}

static inline unsigned grid_for(int64_t n, int64_t per = 256) {
    return (unsigned)std::max<int64_t>(1, std::min<int64_t>(ceil_div(n, per), 1 << 16));
}

template <bool BT>
static rf_status dgemm(hipStream_t s, int64_t M, int64_t N, int64_t K, double alpha, const double* A, int64_t lda,
                       const double* B, int64_t ldb, double beta, double* C, int64_t ldc) {
    if (M <= 0 || N <= 0) return RF_OK;
    hipLaunchKernelGGL(k_dgemm<BT>, dim3((unsigned)ceil_div(M, 64), (unsigned)ceil_div(N, 64)), dim3(256), 0, s, M, N,
                       K, alpha, A, lda, B, ldb, beta, C, ldc);
    return check_launch("rf_solve: dgemm");
}

#define RF_TRY(expr)                      \
    do {                                  \
        rf_status _st = (expr);           \
        if (_st != RF_OK) return _st;     \
    } while (0)

// R (rows x d, ld d) <- R C^-1 using L (in C's lower triangle) and the diagonal inverses.
static rf_status apply_inverse(hipStream_t s, const SolveWs& w, int64_t d, double* R, int64_t rows) {
    const int nblk = (int)(d / kNB);
    // forward:  Z L^T = R
    for (int J = 0; J < nblk; ++J) {
        const int64_t c0 = (int64_t)J * kNB;
        RF_TRY(dgemm<true>(s, rows, kNB, kNB, 1.0, R + c0, d, w.Dinv + c0 * kNB, kNB, 0.0, w.P, kNB));
        hipLaunchKernelGGL(k_copy2d, dim3(grid_for(rows * kNB)), dim3(256), 0, s, w.P, (int64_t)kNB, R + c0, d, rows,
                           (int64_t)kNB);
        RF_TRY(check_launch("rf_solve: copy"));
        const int64_t rem = d - c0 - kNB;
        RF_TRY(dgemm<true>(s, rows, rem, kNB, -1.0, w.P, kNB, w.C + (c0 + kNB) * d + c0, d, 1.0, R + c0 + kNB, d));
    }
    // backward: W L = Z
    for (int J = nblk - 1; J >= 0; --J) {
        const int64_t c0 = (int64_t)J * kNB;
        RF_TRY(dgemm<false>(s, rows, kNB, kNB, 1.0, R + c0, d, w.Dinv + c0 * kNB, kNB, 0.0, w.P, kNB));
        hipLaunchKernelGGL(k_copy2d, dim3(grid_for(rows * kNB)), dim3(256), 0, s, w.P, (int64_t)kNB, R + c0, d, rows,
                           (int64_t)kNB);
        RF_TRY(check_launch("rf_solve: copy"));
        RF_TRY(dgemm<false>(s, rows, c0, kNB, -1.0, w.P, kNB, w.C + c0 * d, d, 1.0, R, d));
    }
    return RF_OK;
}

}  // namespace rf

using namespace rf;

extern "C" {

size_t rf_solve_workspace_bytes(const rf_gram_desc* desc, int32_t n_sel) {
    if (!desc || desc->d <= 0 || desc->d % 256 != 0 || n_sel < 0) return 0;
    return solve_ws(nullptr, desc->d, n_sel).total;
}

rf_status rf_solve(const rf_gram_desc* desc, const void* d_state, double lambda, rf_lambda_mode mode,
                   const int32_t* targets, int32_t n_sel, float* d_W, void* d_W_lp, float* d_b, int32_t* d_info,
                   void* d_ws, size_t ws_bytes, void* stream) {
    clear_error();
    rf_gram_layout_t GL;
    rf_status st = rf_gram_state_layout(desc, &GL);
    if (st != RF_OK) return st;
    RF_REQUIRE(d_state && aligned(d_state, 256), RF_ERR_INVALID_ARG, "rf_solve: state must be non-null, 256-B aligned");
    RF_REQUIRE(d_info, RF_ERR_INVALID_ARG, "rf_solve: null info");
    RF_REQUIRE(isfinite(lambda) && lambda >= 0.0, RF_ERR_INVALID_ARG, "rf_solve: lambda must be finite and >= 0");
    RF_REQUIRE(mode == RF_LAMBDA_ABSOLUTE || mode == RF_LAMBDA_REL_MEAN_DIAG, RF_ERR_INVALID_ARG, "rf_solve: bad lambda mode");
    RF_REQUIRE(n_sel >= 0 && n_sel <= kMaxSel, RF_ERR_UNSUPPORTED, "rf_solve: 0..64 selected targets");
    RF_REQUIRE(n_sel == 0 || targets, RF_ERR_INVALID_ARG, "rf_solve: null targets");
    for (int i = 0; i < n_sel; ++i)
        RF_REQUIRE(targets[i] >= 0 && targets[i] < desc->n_targets, RF_ERR_INVALID_ARG, "rf_solve: target index out of range");
    RF_REQUIRE(aligned(d_ws, 256), RF_ERR_INVALID_ARG, "rf_solve: workspace must be 256-B aligned");
    const int64_t d = desc->d;
    const SolveWs w = solve_ws(d_ws, d, n_sel);
    RF_REQUIRE(d_ws && ws_bytes >= w.total, RF_ERR_WORKSPACE, "rf_solve: workspace too small");
    hipStream_t s = (hipStream_t)stream;
    const char* sp = (const char*)d_state;
    const float* Sxx = (const float*)(sp + GL.off_S_xx);
    const float* Syx = (const float*)(sp + GL.off_S_yx);
    const double* sx = (const double*)(sp + GL.off_s_x);
    const double* sy = (const double*)(sp + GL.off_s_y);
    const int64_t* np = (const int64_t*)(sp + GL.off_n);

    hipLaunchKernelGGL(k_zero_int, dim3(1), dim3(1), 0, s, d_info);
    RF_TRY(check_launch("rf_solve: info"));
    hipLaunchKernelGGL(k_centre_gram, dim3(grid_for(d * d)), dim3(256), 0, s, Sxx, sx, np, d, w.C);
    RF_TRY(check_launch("rf_solve: centre"));
    hipLaunchKernelGGL(k_add_lambda, dim3(1), dim3(256), 0, s, w.C, d, lambda, (int)(mode == RF_LAMBDA_REL_MEAN_DIAG));
    RF_TRY(check_launch("rf_solve: lambda"));

    // blocked Cholesky
    const int nblk = (int)(d / kNB);
    for (int J = 0; J < nblk; ++J) {
        const int64_t c0 = (int64_t)J * kNB;
        hipLaunchKernelGGL(k_chol_diag, dim3(1), dim3(256), 0, s, w.C, d, J, w.Dinv, d_info);
        RF_TRY(check_launch("rf_solve: potrf"));
        const int64_t rem = d - c0 - kNB;
        if (rem <= 0) continue;
        double* panel = w.C + (c0 + kNB) * d + c0;
        RF_TRY(dgemm<true>(s, rem, kNB, kNB, 1.0, panel, d, w.Dinv + c0 * kNB, kNB, 0.0, w.P, kNB));
        RF_TRY(dgemm<true>(s, rem, rem, kNB, -1.0, w.P, kNB, w.P, kNB, 1.0, w.C + (c0 + kNB) * d + c0 + kNB, d));
        hipLaunchKernelGGL(k_copy2d, dim3(grid_for(rem * kNB)), dim3(256), 0, s, w.P, (int64_t)kNB, panel, d, rem,
                           (int64_t)kNB);
        RF_TRY(check_launch("rf_solve: copy"));
    }
    // C^-1 by the two triangular solves on the identity
    hipLaunchKernelGGL(k_identity, dim3(grid_for(d * d)), dim3(256), 0, s, w.Cinv, d);
    RF_TRY(check_launch("rf_solve: identity"));
    RF_TRY(apply_inverse(s, w, d, w.Cinv, d));
    if (n_sel == 0) return RF_OK;

    const int64_t rows = (int64_t)n_sel * d;
    CrossArgs ca{};
    ca.Syx = Syx; ca.sy = sy; ca.sx = sx; ca.np = np; ca.d = d; ca.rows = rows; ca.R = w.R; ca.mu_y = w.mu_y;
    for (int i = 0; i < n_sel; ++i) ca.tsel[i] = targets[i];
    hipLaunchKernelGGL(k_centre_cross, dim3(grid_for(rows * d)), dim3(256), 0, s, ca);
    RF_TRY(check_launch("rf_solve: centre cross"));
    // W = B C^-1 (C^-1 symmetric, so its rows serve as columns)
    RF_TRY(dgemm<true>(s, rows, d, d, 1.0, w.R, d, w.Cinv, d, 0.0, w.W, d));
    if (d_b) {
        hipLaunchKernelGGL(k_bias, dim3((unsigned)ceil_div(rows, 4)), dim3(256), 0, s, w.W, sx, np, w.mu_y, d, rows, d_b);
        RF_TRY(check_launch("rf_solve: bias"));
    }
    if (d_W || d_W_lp) {
        hipLaunchKernelGGL(k_store_w, dim3(grid_for(rows * d)), dim3(256), 0, s, w.W, rows * d, d_W, (bf16_t*)d_W_lp);
        RF_TRY(check_launch("rf_solve: store"));
    }
    return RF_OK;
}

}  // extern "C"
