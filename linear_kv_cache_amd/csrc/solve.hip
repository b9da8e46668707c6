// Closed-form ridge solve from the one-pass statistics (RidgeFill project page, "Method"
// step 2: a ridge regression fitted once in closed form; intercept by mean-centring).
//
//   A  = S_xx - s_x^T s_x / n + lambda I           fp64, symmetric from the upper triangle
//   A = L L^T                                      blocked right-looking Cholesky, 64-wide panels
//   Z = L^-T, A^-1 = Z Z^T                          blocked forward solve on the identity, one GEMM
//   B  = S_yx,l - s_y,l^T s_x / n                  fp64 per element, one row per (target, output)
//   W  = B A^-1,  b = s_y/n - W (s_x/n)
// The large product W = B A^-1 ([n_sel d] x d x d) runs on the bf16 MFMA pipes in three-term
// split precision: with D = diag(A), W = (B D^-1/2)(D^1/2 A^-1 D^1/2) D^-1/2, and each
// equilibrated factor F is split into bf16 parts F = F_hi + F_lo, so that
//   W D^1/2 = B_hi Ah + B_hi Al + B_lo Ah        (the F_lo x F_lo term is below fp32 rounding)
// accumulated in fp32.  The equilibrated inverse has unit-scale entries and a condition
// number near that of the data's correlation matrix, so the result matches the fp64 product
// to ~1e-5 of max |W|.  Diagonal 64 x 64 blocks are factored and inverted by one wave each;
// the blocked updates are tiled fp64 GEMMs.  All reductions run in a fixed order.
#include <math.h>

#include "rf_internal.h"
#include "rf_mfma.h"
#include "rf_pipe.h"

namespace rf {

constexpr int kNB = 64;        // Cholesky / triangular-solve block
constexpr int kMaxSel = 64;

// ---- tiled fp64 GEMM on the matrix cores:  C = alpha * A * op(B) + beta * C ----------------
// A [M][K] (lda); op(B) = B^T with B [N][K] (BT) or B [K][N] (!BT); beta == 0 never reads C.
// 128 x 128 tile per work-group of 4 waves (2 x 2), each wave 64 x 64 as 4 x 4 blocks of
// v_mfma_f64_16x16x4_f64 (lane l: A[l % 16][k0 + l / 16], B[k0 + l / 16][l % 16]; accumulator
// element r of lane l is C[4 r + l / 16][l % 16], as measured on gfx950).  k-slices of 16 are staged in LDS as
// [k][m] and [k][n], double-buffered; out-of-range rows and columns read as zero.
typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef double f64x2 __attribute__((ext_vector_type(2)));

// Structure flags: kLowerOnly skips tiles wholly above the diagonal (the caller reads only the
// lower triangle of C); kUpperOperands means A and B are upper triangular (A[m][k] = B[n][k] = 0
// for k < m, k < n), so a tile's k-loop starts at max(m0, n0); kUpperA means only A is upper
// triangular (the k-loop starts at m0); kUpperB means B, given as [K][N], is upper triangular
// (B[k][n] = 0 for k > n: the k-loop ends at n0 + BN).
// The flags are bits and combine.
// Batched launches (gridDim.z > 1) offset A, B and C by blockIdx.z times sA, sB, sC elements.
// ``gate`` (device, may be null): the launch does nothing when *gate is 0.
enum { kFull = 0, kLowerOnly = 1, kUpperOperands = 2, kUpperA = 4, kUpperB = 8 };

// One tile (bx, by) of product bz; the whole work-group takes part (it has barriers).
template <bool BT, int BM>
__device__ __attribute__((always_inline)) inline void dgemm_tile(int64_t bx, int64_t by, int64_t bz, int64_t M, int64_t N, int64_t K, double alpha,
                                  const double* A, int64_t lda, const double* B, int64_t ldb, double beta, double* C,
                                  int64_t ldc, int structure, int64_t sA, int64_t sB, int64_t sC) {
    static_assert(BM == 64 || BM == 128, "64 x 64 or 128 x 128 tiles");
    constexpr int BN = BM, BK = 16, PAD = 2;
    constexpr int WT = BM / 2, WB = WT / 16;   // wave tile and its 16 x 16 blocks per side
    // Loads are 16-byte chunks, and each wave instruction covers whole operand rows (coalesced).
    // K-contiguous operands (A, and B when BT) stay row-major in LDS, [m][BK + 2]: the 144-byte
    // row stride is 16-byte aligned for the stores and puts the 16 rows a fragment read touches
    // (plus the next k's 16 lanes) on distinct banks.  An N-contiguous B stays [k][BN + 2].
    // 16-wide k-steps keep a 128 x 128 tile's two LDS stages at 72 KiB and the registers under
    // 256, so two work-groups share a CU and hide each other's load and LDS latency.
    constexpr int CPR_K = BK / 2, RPP_K = 256 / CPR_K, PK = BM / RPP_K;   // chunks/row, rows/pass, passes
    constexpr int CPR_N = BN / 2, RPP_N = 256 / CPR_N, PN = BK / RPP_N;
    constexpr int PB = BT ? PK : PN;
    A += bz * sA;
    B += bz * sB;
    C += bz * sC;
    __shared__ __attribute__((aligned(16))) double As[2][BM][BK + PAD];
    __shared__ __attribute__((aligned(16))) double Bs[2][BT ? BN : BK][BT ? BK + PAD : BN + PAD];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t m0 = bx * BM, n0 = by * BN;
    if ((structure & kLowerOnly) && n0 > m0 + BM - 1) return;
    int64_t kbeg = 0, kend = K;
    if (structure & kUpperOperands) kbeg = (m0 > n0 ? m0 : n0) / BK * BK;
    if (structure & kUpperA) kbeg = m0 / BK * BK;
    if ((structure & kUpperB) && n0 + BN < K) kend = n0 + BN;
    f64x2 ra[PK], rb[PB];
    // two consecutive elements of a row; a pair wholly in range and 16-byte aligned is one load
    auto pair = [&](const double* row, bool row_ok, int64_t c, int64_t lim) -> f64x2 {
        const double* q = row + c;
        if (row_ok && c + 1 < lim && ((uintptr_t)q & 15) == 0) return *(const f64x2*)q;
        return f64x2{row_ok && c < lim ? q[0] : 0.0, row_ok && c + 1 < lim ? q[1] : 0.0};
    };
    auto load = [&](int64_t k0) {
        const int64_t kc = k0 + 2 * (t % CPR_K);
#pragma unroll
        for (int u = 0; u < PK; ++u) {
            const int64_t m = m0 + t / CPR_K + RPP_K * u;
            ra[u] = pair(A + (m < M ? m : 0) * lda, m < M, kc, K);
        }
        if (BT) {
#pragma unroll
            for (int u = 0; u < PK; ++u) {
                const int64_t n = n0 + t / CPR_K + RPP_K * u;
                rb[u] = pair(B + (n < N ? n : 0) * ldb, n < N, kc, K);
            }
        } else {
            const int64_t nc = n0 + 2 * (t % CPR_N);
#pragma unroll
            for (int u = 0; u < PN; ++u) {
                const int64_t k = k0 + t / CPR_N + RPP_N * u;
                rb[u] = pair(B + (k < K ? k : 0) * ldb, k < K, nc, N);
            }
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int u = 0; u < PK; ++u) *(f64x2*)&As[buf][t / CPR_K + RPP_K * u][2 * (t % CPR_K)] = ra[u];
        if (BT) {
#pragma unroll
            for (int u = 0; u < PK; ++u) *(f64x2*)&Bs[buf][t / CPR_K + RPP_K * u][2 * (t % CPR_K)] = rb[u];
        } else {
#pragma unroll
            for (int u = 0; u < PN; ++u) *(f64x2*)&Bs[buf][t / CPR_N + RPP_N * u][2 * (t % CPR_N)] = rb[u];
        }
    };
    f64x4 acc[WB][WB];
#pragma unroll
    for (int i = 0; i < WB; ++i)
#pragma unroll
        for (int j = 0; j < WB; ++j) acc[i][j] = f64x4{0.0, 0.0, 0.0, 0.0};
    const int nk = kend > kbeg ? (int)((kend - kbeg + BK - 1) / BK) : 0;
    if (nk > 0) {
        load(kbeg);
        store(0);
        __syncthreads();
        for (int kt = 0; kt < nk; ++kt) {
            const int cur = kt & 1;
            if (kt + 1 < nk) load(kbeg + (int64_t)(kt + 1) * BK);
#pragma unroll
            for (int ks = 0; ks < BK; ks += 4) {
                const int kr = ks + (lane >> 4);
                double a[WB], b[WB];
#pragma unroll
                for (int i = 0; i < WB; ++i) a[i] = As[cur][wm * WT + i * 16 + (lane & 15)][kr];
#pragma unroll
                for (int j = 0; j < WB; ++j)
                    b[j] = BT ? Bs[cur][wn * WT + j * 16 + (lane & 15)][kr] : Bs[cur][kr][wn * WT + j * 16 + (lane & 15)];
#pragma unroll
                for (int i = 0; i < WB; ++i)
#pragma unroll
                    for (int j = 0; j < WB; ++j) acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], b[j], acc[i][j], 0, 0, 0);
            }
            if (kt + 1 < nk) store(cur ^ 1);
            __syncthreads();
        }
    }
    // all reads of C before any write (a store followed by a load the compiler cannot prove
    // disjoint would otherwise cost a full memory round trip per element), half a tile at a time
#pragma unroll
    for (int ih = 0; ih < WB; ih += WB / 2) {
        double cv[WB / 2][WB][4];
#pragma unroll
        for (int i = 0; i < WB / 2; ++i)
#pragma unroll
            for (int j = 0; j < WB; ++j) {
                const int64_t n = n0 + wn * WT + j * 16 + (lane & 15);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int64_t m = m0 + wm * WT + (ih + i) * 16 + 4 * r + (lane >> 4);
                    cv[i][j][r] = (beta != 0.0 && m < M && n < N) ? C[m * ldc + n] : 0.0;
                }
            }
#pragma unroll
        for (int i = 0; i < WB / 2; ++i) {
#pragma unroll
            for (int j = 0; j < WB; ++j) {
                const int64_t n = n0 + wn * WT + j * 16 + (lane & 15);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int64_t m = m0 + wm * WT + (ih + i) * 16 + 4 * r + (lane >> 4);
                    if (m < M && n < N) {
                        double v = alpha * acc[ih + i][j][r];
                        if (beta != 0.0) v += beta * cv[i][j][r];
                        C[m * ldc + n] = v;
                    }
                }
            }
        }
    }
}

template <bool BT, int BM = 128>
__global__ __launch_bounds__(256, 2) void k_dgemm(int64_t M, int64_t N, int64_t K, double alpha, const double* A,
                                               int64_t lda, const double* B, int64_t ldb, double beta, double* C,
                                               int64_t ldc, int structure, int64_t sA, int64_t sB, int64_t sC,
                                               const int32_t* gate) {
    if (gate && *gate == 0) return;   // a conditional product that is not wanted
    dgemm_tile<BT, BM>(blockIdx.x, blockIdx.y, blockIdx.z, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, structure,
                       sA, sB, sC);
}

// Z = 0 except its diagonal 64 x 64 blocks, which are the transposed inverses of L's diagonal
// blocks (Dinv holds L_JJ^-1 row-major): Z_JJ = (L_JJ^T)^-1.
__global__ void k_zdiag(const double* Dinv, int64_t d, double* Z) {
    const int64_t n = d * d;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = i / d, c = i % d;
        const int64_t J = r / kNB;
        Z[i] = c / kNB == J ? Dinv[(J * kNB + c % kNB) * kNB + r % kNB] : 0.0;
    }
}

__global__ void k_zero_int(int32_t* p, int n) {
    if ((int)threadIdx.x < n) p[threadIdx.x] = 0;
}

// Head-wise maps: with hdim > 0, feature i belongs to head (i % hper) / hdim (hper = the
// targets' width; the sources are whole multiples of it), and the centred moments between
// different heads are taken as zero, so the system is block-diagonal by head.
__device__ inline bool cross_head(int32_t hdim, int32_t hper, int64_t i, int64_t j) {
    return hdim > 0 && (i % hper) / hdim != (j % hper) / hdim;
}

// C[i][j] = S_xx[min(i,j)][max(i,j)] - s_x[i] s_x[j] / n (0 between heads), into every matrix
// of the batch (blockIdx.y: one per lambda, d*d elements apart)
__global__ void k_centre_gram(const float* Sxx, const double* sx, const int64_t* np, int64_t d, double* C,
                              int32_t hdim, int32_t hper) {
    C += (int64_t)blockIdx.y * d * d;
    const double inv_n = 1.0 / (double)*np;
    const int64_t n = d * d;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n; idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t i = idx / d, j = idx % d;
        const int64_t lo = i < j ? i : j, hi = i < j ? j : i;
        C[idx] = cross_head(hdim, hper, i, j) ? 0.0 : (double)Sxx[lo * d + hi] - sx[i] * sx[j] * inv_n;
    }
}

constexpr int kMaxLambda = 8;
struct Lambdas {
    double v[kMaxLambda];
};

// Adds lambda (absolute, or times the mean diagonal) to the diagonal: one work-group per
// matrix of the batch (blockIdx.x; d*d elements apart), lambda lam.v[blockIdx.x].
__global__ __launch_bounds__(256) void k_add_lambda(double* C, int64_t d, Lambdas lams, int rel) {
    __shared__ double red[256];
    C += (int64_t)blockIdx.x * d * d;
    const double lambda = lams.v[blockIdx.x];
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

// v = hi + lo with hi = bf16(v) and lo = bf16(v - hi) (each rounded to nearest even; the
// double rounding through fp32 is exact for hi's bf16 grid and below lo's precision).
__device__ inline void split_bf16(double v, bf16_t& hi, bf16_t& lo) {
    const __bf16 h = (__bf16)(float)v;
    hi = __builtin_bit_cast(uint16_t, h);
    lo = __builtin_bit_cast(uint16_t, (__bf16)(float)(v - (double)(float)h));
}

struct CrossArgs {
    const float* Syx;
    const double* sy;
    const double* sx;
    const int64_t* np;
    const double* rdg;     // 1 / sqrt(diag(C + lambda I))
    int64_t d;
    int64_t dy;            // outputs per target
    int64_t rows;          // n_sel * dy
    bf16_t* Aq;            // [rows][2d]: [hi | lo] of the equilibrated centred cross moments
    double* mu_y;          // [rows]
    int32_t hdim, hper;    // head-wise maps (hdim > 0): moments between heads taken as zero
    int32_t tsel[kMaxSel];
};

// Centred cross moments B[c][i] = S_yx[c][i] - s_y[c] s_x[i] / n (fp64), scaled by rdg[i] = 1/dg[i]
// and split into bf16 parts: the 8 consecutive columns i0 .. i0 + 7 of row c (16-byte stores).
// Runs in the spare work-groups of the diagonal-block launches (below): it does not depend on
// the factorisation, and those launches otherwise leave all but one CU idle.
__device__ inline void centre_split_row(const CrossArgs& a, int64_t c, int64_t i0) {
    const double inv_n = 1.0 / (double)*a.np;
    const int64_t s = c / a.dy, o = c - s * a.dy;
    const int64_t srow = (int64_t)a.tsel[s] * a.dy + o;
    const double syv = a.sy[srow];
    const f32x4 v0 = *(const f32x4*)(a.Syx + srow * a.d + i0);
    const f32x4 v1 = *(const f32x4*)(a.Syx + srow * a.d + i0 + 4);
    // the 8 columns lie in one head (head widths are multiples of 8)
    const double keep = cross_head(a.hdim, a.hper, o, i0) ? 0.0 : 1.0;
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
        bf16_t h0, l0, h1, l1;
        const float x0 = e < 4 ? v0[e] : v1[e - 4], x1 = e < 4 ? v0[e + 1] : v1[e - 3];
        split_bf16(keep * (((double)x0 - syv * a.sx[i0 + e] * inv_n) * a.rdg[i0 + e]), h0, l0);
        split_bf16(keep * (((double)x1 - syv * a.sx[i0 + e + 1] * inv_n) * a.rdg[i0 + e + 1]), h1, l1);
        hi[e / 2] = (uint32_t)h0 | ((uint32_t)h1 << 16);
        lo[e / 2] = (uint32_t)l0 | ((uint32_t)l1 << 16);
    }
    bf16_t* row = a.Aq + c * 2 * a.d;
    *(u32x4*)(row + i0) = u32x4{hi[0], hi[1], hi[2], hi[3]};
    *(u32x4*)(row + a.d + i0) = u32x4{lo[0], lo[1], lo[2], lo[3]};
    if (i0 == 0) a.mu_y[c] = syv * inv_n;
}

// A double held by lane ``lane`` (a compile-time constant here) as a wave-uniform value.
__device__ inline double readlane_f64(double x, int lane) {
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), lane);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// sqrt(p) and 1/sqrt(p) from the hardware reciprocal square root refined by two Newton steps
// (y <- y + y (1 - p y^2) / 2, each doubling the correct bits) and a final Newton step on the
// square root itself (r <- r + (p - r^2) y / 2).  Non-positive p gives a non-finite pair.
__device__ inline void sqrt_rsqrt(double p, double& r, double& ri) {
    double y = __builtin_amdgcn_rsq(p);
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const double e = fma(-(p * y), y, 1.0);
        y = fma(0.5 * y, e, y);
    }
    double s = p * y;
    s = fma(0.5 * y, fma(-s, s, p), s);
    r = s;
    ri = y;
}

// Factor the diagonal block J (already updated by all earlier panels) in place into L_JJ and
// write L_JJ^-1 into Dinv.  info receives the 1-based index of the first non-positive pivot
// (unless an earlier block already reported one).
// One wave, no barriers (a wave's LDS operations complete in order).  Lane i keeps row i of the
// block in registers.  Right-looking elimination: at step j lane i scales its entry of column j
// by the pivot's inverse square root and writes L[i][j] into the transposed copy Lt[j][i]; the
// multipliers L[k][j] then reach every lane as broadcast reads of Lt[j] (all lanes one address).
// The step's critical path stays in registers: the next column's entry is updated first with
// L[j+1][j] read across lanes, and the next pivot is read from lane j+1 the same way, so its
// square root overlaps the rest of step j's update.  Entries above the diagonal are never read
// for the lower triangle and are written as zeros.  L^-1 by right-looking substitution, lane c
// holding column c: once X[k][c] is final it is stored, and row k of X updates the running sums
// of rows r > k with L[r][k] = Lt[k][r].
// Called by the first wave of a work-group only.
__device__ __attribute__((always_inline)) inline void chol_diag_block(double* C, int64_t d, int J, double* Dinv, int32_t* info) {
    __shared__ __attribute__((aligned(16))) double Lt[kNB][kNB + 2];
    const int i = threadIdx.x;
    const int64_t off = (int64_t)J * kNB;
    double a[kNB];
#pragma unroll
    for (int k = 0; k < kNB; ++k) a[k] = C[(off + i) * d + off + k];
    const bool prior = *info != 0;
    int32_t fail = 0;
    double rinv = 0.0;   // lane i: 1 / L[i][i]
    double r, ri;        // sqrt of the current pivot and its inverse (wave-uniform)
    {
        const double p = readlane_f64(a[0], 0);
        if (!(p > 0.0)) fail = (int32_t)(off + 1);
        sqrt_rsqrt(p, r, ri);
    }
#pragma unroll
    for (int j = 0; j < kNB; ++j) {
        const double lij = i > j ? a[j] * ri : (i == j ? r : 0.0);
        if (i == j) rinv = ri;
        Lt[j][i] = lij;
        a[j] = i >= j ? lij : a[j];
        double rn = 0.0, rin = 0.0;
        if (j + 1 < kNB) {
            // next column first: L[j+1][j] from lane j+1, then the next pivot from lane j+1
            a[j + 1] -= lij * readlane_f64(lij, j + 1);
            const double pn = readlane_f64(a[j + 1], j + 1);
            if (!(pn > 0.0) && fail == 0) fail = (int32_t)(off + j + 2);
            sqrt_rsqrt(pn, rn, rin);
        }
        int k0 = j + 2;
        if ((k0 & 1) && k0 < kNB) {
            a[k0] -= lij * Lt[j][k0];
            ++k0;
        }
#pragma unroll
        for (int k = k0; k < kNB; k += 2) {
            const f64x2 v = *(const f64x2*)(&Lt[j][k]);   // broadcast of L[k][j], L[k+1][j]
            a[k] -= lij * v[0];
            a[k + 1] -= lij * v[1];
        }
        r = rn;
        ri = rin;
        __builtin_amdgcn_sched_barrier(0);   // one step per scheduling region
    }
#pragma unroll
    for (int k = 0; k < kNB; ++k) C[(off + i) * d + off + k] = k <= i ? a[k] : 0.0;
    if (i == 0 && !prior && fail != 0) *info = fail;
    // 1 / L[k][k] is lane k's rinv, read across lanes (no LDS round trip on the chain)
    double* D = Dinv + (int64_t)J * kNB * kNB;
    double acc[kNB];   // lane c: sum_{k < r, so far} L[r][k] X[k][c]
#pragma unroll
    for (int r = 0; r < kNB; ++r) acc[r] = 0.0;
#pragma unroll
    for (int k = 0; k < kNB; ++k) {
        const double xk = ((k == i ? 1.0 : 0.0) - acc[k]) * readlane_f64(rinv, k);
        D[k * kNB + i] = xk;
        if ((k & 1) == 0 && k + 1 < kNB) acc[k + 1] += Lt[k][k + 1] * xk;
#pragma unroll
        for (int r = (k + 2) & ~1; r < kNB; r += 2) {
            const f64x2 v = *(const f64x2*)(&Lt[k][r]);   // broadcast of L[r][k], L[r+1][k]
            acc[r] += v[0] * xk;
            acc[r + 1] += v[1] * xk;
            if ((r & 15) == 14) __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Work-group z < n_lam factors the block of matrix z (C + z sC, Dinv + z sD, info + z) with
// its first wave; the work-groups after those centre and split rows [c_begin, c_end) of the
// cross moments, ny work-groups of 2048 columns per row.
__global__ __launch_bounds__(256) void k_chol_diag(double* C, int64_t sC, int64_t d, int J, double* Dinv, int64_t sD,
                                                   int32_t* info, int n_lam, CrossArgs ca, int64_t c_begin,
                                                   int64_t c_end, int ny) {
    if ((int)blockIdx.x >= n_lam) {
        const int64_t b = blockIdx.x - n_lam;
        const int64_t c = c_begin + b / ny;
        const int64_t i0 = ((b % ny) * 256 + threadIdx.x) * 8;
        if (c < c_end && i0 < ca.d) centre_split_row(ca, c, i0);
        return;
    }
    if (threadIdx.x >= 64) return;   // the factorisation is one wave's (no barriers in it)
    chol_diag_block(C + (int64_t)blockIdx.x * sC, d, J, Dinv + (int64_t)blockIdx.x * sD, info + blockIdx.x);
}

// The rest of a step's trailing update: P = the step's panel rows below the next block (ld d),
// C = the trailing matrix below and right of the next block, m x m, lower 64 x 64 tiles only
// (tiles of them per matrix, in the order t = bx (bx + 1) / 2 + by, by <= bx).
struct TrailArgs {
    const double* P;
    double* C;
    int64_t m;
    int64_t tiles;
};

// Step J of the blocked Cholesky beside the end of step J - 1: block column J was updated by
// step J - 1 first, so its diagonal block (work-groups z < n_lam, as k_chol_diag) is factored
// in the same launch as the rest of step J - 1's trailing update (the next tiles x n_lam
// work-groups; those never touch block row or column J), then the centring slices.
__global__ __launch_bounds__(256, 2) void k_chol_step(double* C, int64_t sC, int64_t d, int J, double* Dinv,
                                                      int64_t sD, int32_t* info, int n_lam, TrailArgs u, CrossArgs ca,
                                                      int64_t c_begin, int64_t c_end, int ny) {
    int64_t b = blockIdx.x;
    if (b < n_lam) {
        if (threadIdx.x < 64) chol_diag_block(C + b * sC, d, J, Dinv + b * sD, info + b);
        return;
    }
    b -= n_lam;
    if (b < u.tiles * n_lam) {
        const int64_t z = b / u.tiles, t = b % u.tiles;
        int64_t bx = (int64_t)((sqrt(8.0 * (double)t + 1.0) - 1.0) * 0.5);
        while (bx * (bx + 1) / 2 > t) --bx;
        while ((bx + 1) * (bx + 2) / 2 <= t) ++bx;
        const int64_t by = t - bx * (bx + 1) / 2;
        dgemm_tile<true, 64>(bx, by, z, u.m, u.m, kNB, -1.0, u.P, d, u.P, d, 1.0, u.C, d, kLowerOnly, sC, sC, sC);
        return;
    }
    b -= u.tiles * n_lam;
    const int64_t c = c_begin + b / ny;
    const int64_t i0 = ((b % ny) * 256 + threadIdx.x) * 8;
    if (c < c_end && i0 < ca.d) centre_split_row(ca, c, i0);
}

// dg[i] = sqrt(A[i][i]) before the factorisation overwrites the diagonal, and rdg[i] = 1/dg[i]
// (the unscaling steps multiply by it instead of dividing).  A zero diagonal (a feature with
// no variance: only the pseudo-inverse route gets that far) keeps the scale 1.
__global__ void k_diag_sqrt(const double* A, int64_t d, double* dg, double* rdg) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < d) {
        const double a = fabs(A[i * d + i]);
        dg[i] = a > 0.0 ? sqrt(a) : 1.0;
        rdg[i] = 1.0 / dg[i];
    }
}

// Equilibrated inverse, split: row j of Bq = [hi | lo | hi] of Ainv[j][i] dg[i] dg[j], stored in
// the packed fragment order of the W product's weight operand (K = 3d columns).
// One 64 x 64 tile of A^-1 per work-group.  Only the lower triangle of A^-1 (by 64-blocks) is
// formed; a tile above the diagonal reads its mirror image (coalesced) and transposes it
// through LDS.  Each thread then splits 8 consecutive columns of one row and stores them as
// three 16-byte fragment chunks.  hmax (may be null) receives the tile's largest |entry| of the
// equilibrated inverse, at [blockIdx.y][blockIdx.x].
__global__ __launch_bounds__(256) void k_split_inverse(const double* Ainv, const double* dg, int64_t d, bf16_t* Bq,
                                                       double* hmax) {
    __shared__ double tile[64][65];
    __shared__ double red[256];
    double hm = 0.0;
    bool bad = false;   // a NaN entry (fmax would drop it)
    const int64_t ib = blockIdx.x, jb = blockIdx.y;   // element (j, i): Bq row j, column i
    const bool mirror = ib > jb;
    const int64_t r0 = (mirror ? ib : jb) * 64, c0 = (mirror ? jb : ib) * 64;
    for (int e = threadIdx.x; e < 64 * 64; e += 256) tile[e / 64][e % 64] = Ainv[(r0 + e / 64) * d + c0 + e % 64];
    __syncthreads();
    const int64_t K = 3 * d;
    for (int e = threadIdx.x; e < 64 * 8; e += 256) {
        const int jl = e >> 3, i8 = (e & 7) * 8;
        const int64_t j = jb * 64 + jl, i0 = ib * 64 + i8;
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int il = i8 + 2 * q;
            bf16_t h0, l0, h1, l1;
            const double v0 = (mirror ? tile[il][jl] : tile[jl][il]) * dg[i0 + 2 * q] * dg[j];
            const double v1 = (mirror ? tile[il + 1][jl] : tile[jl][il + 1]) * dg[i0 + 2 * q + 1] * dg[j];
            hm = fmax(hm, fmax(fabs(v0), fabs(v1)));
            bad |= (v0 != v0) || (v1 != v1);
            split_bf16(v0, h0, l0);
            split_bf16(v1, h1, l1);
            hi[q] = (uint32_t)h0 | ((uint32_t)h1 << 16);
            lo[q] = (uint32_t)l0 | ((uint32_t)l1 << 16);
        }
        const u32x4 H{hi[0], hi[1], hi[2], hi[3]}, Lo{lo[0], lo[1], lo[2], lo[3]};
        *(u32x4*)(Bq + packed_index(j, (int)i0, K)) = H;
        *(u32x4*)(Bq + packed_index(j, (int)(d + i0), K)) = Lo;
        *(u32x4*)(Bq + packed_index(j, (int)(2 * d + i0), K)) = H;
    }
    if (hmax) {
        red[threadIdx.x] = bad ? INFINITY : hm;
        __syncthreads();
        for (int h = 128; h > 0; h >>= 1) {
            if ((int)threadIdx.x < h) red[threadIdx.x] = fmax(red[threadIdx.x], red[threadIdx.x + h]);
            __syncthreads();
        }
        if (threadIdx.x == 0) hmax[(int64_t)blockIdx.y * gridDim.x + blockIdx.x] = red[0];
    }
}

// W = Aq Bq^T over K = 3d.  MFMA operand A = Bq rows (input feature j), B = Aq rows
// (output c), so each lane holds 4 consecutive j of one c: W[c][j..j+3] = acc rdg[j] is one
// 16-byte (fp32) and one 8-byte (bf16) store.  The epilogue also leaves, per (c, tile of 256
// j), the partial dot  sum_j W[c][j] s_x[j] / n  for the bias.
struct WArgs {
    const bf16_t* Aq;
    const bf16_t* Bq;
    const double* rdg;
    const double* sx;
    const int64_t* np;
    int64_t d;
    int64_t rows;
    int32_t tiles_j;
    int32_t tiles_c;
    float* W;          // may be null
    bf16_t* Wlp;       // may be null
    float* bpart;      // [rows][tiles_j]
};

__global__ __launch_bounds__(PackedAGemm::kThr) void k_wgemm(WArgs a) {
    using G = PackedAGemm;   // Bq arrives packed (k_split_inverse)
    __shared__ __attribute__((aligned(16))) char lds[G::LDS_BYTES];
    const int v = xcd_order((int)blockIdx.x, (int)gridDim.x);
    int jt, ct;
    grouped_tile(v, a.tiles_j, a.tiles_c, 4, jt, ct);
    const int64_t j0 = (int64_t)jt * 256, c0 = (int64_t)ct * 256;
    const int64_t K = 3 * a.d;
    G gm;
    // Aq rows are [hi | lo] (2d): the k-steps of the three K segments read hi, hi, lo
    gm.run<true>(lds, PipeOperand{a.Bq + j0 * K, K, 256}, PipeOperand{a.Aq + c0 * 2 * a.d, 2 * a.d, a.rows - c0},
                 (int)(K / G::BK), (int)(a.d / G::BK));

    const double inv_n = 1.0 / (double)*a.np;
    const int lane = threadIdx.x & 63;
    constexpr int kWaveRows = G::kThr / 64 / G::WGN;
    const int wm = (threadIdx.x >> 6) / G::WGN;   // wave row
    float* red = (float*)lds;  // [kWaveRows][256]; the main loop ended on a barrier
#pragma unroll
    for (int jb = 0; jb < G::SN; ++jb) {
        const int cl = G::col_of(jb);
        const int64_t c = c0 + cl;
        const int64_t wl_base = c0 * a.d + packed_row_part(cl);
        float part = 0.f;
#pragma unroll
        for (int i = 0; i < G::SM; ++i) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t j = j0 + G::row_of(i, 4 * q);
                float w[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    w[e] = (float)((double)gm.acc[i][jb][4 * q + e] * a.rdg[j + e]);
                    part += w[e] * (float)(a.sx[j + e] * inv_n);
                }
                if (a.W) *(f32x4*)(a.W + c * a.d + j) = f32x4{w[0], w[1], w[2], w[3]};
                // the bf16 map in the fill's packed layout (256-row tiles never straddle targets)
                if (a.Wlp)
                    *(u32x2*)(a.Wlp + wl_base + packed_col_part((int)j)) =
                        u32x2{pack_bf16x2(w[0], w[1]), pack_bf16x2(w[2], w[3])};
            }
        }
        part += __shfl_xor(part, 32);
        if (lane < 32) red[wm * 256 + cl] = part;
    }
    __syncthreads();
    const int cl = threadIdx.x;
    if (cl < 256) {
        float ps = 0.f;
#pragma unroll
        for (int w = 0; w < kWaveRows; ++w) ps += red[w * 256 + cl];
        a.bpart[(c0 + cl) * a.tiles_j + jt] = ps;
    }
}

// b[c] = mu_y[c] - sum over tiles of the partial dots (fixed order, fp64).
__global__ void k_bias(const float* bpart, int tiles_j, const double* mu_y, int64_t rows, float* b) {
    const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= rows) return;
    double s = 0.0;
    for (int t = 0; t < tiles_j; ++t) s += (double)bpart[c * tiles_j + t];
    b[c] = (float)(mu_y[c] - s);
}


// ---- the fp64 route of the W product and the stationarity residual ------------------------
// Each of these does nothing when its gate (device, may be null) holds 0, so a route chosen on
// the device from the conditioning of the system is launched without a host round trip.

// One work-group per d x d tile row pair: the full symmetric A^-1 from its lower triangle
// (element (i, j) with i >= j holds A^-1, as the Z Z^T product leaves it).
__global__ void k_mirror_full(const double* Ainv_lower, int64_t d, double* Afull, const int32_t* gate) {
    if (gate && *gate == 0) return;
    const int64_t n = d * d;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n; idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t i = idx / d, j = idx % d;
        Afull[idx] = i >= j ? Ainv_lower[idx] : Ainv_lower[j * d + i];
    }
}

// Centred cross moments in fp64 for rows [r0, r0 + nr) of the selected targets' outputs, one
// row per work-group at a time (rows strided by the grid, so a gated-off launch stays small):
// Bf[r - r0][i] = S_yx[row][i] - s_y[row] s_x[i] / n; bmax (may be null) receives max_i |Bf| of
// each row at its global row index.
__global__ __launch_bounds__(256) void k_centre_f64(CrossArgs a, int64_t r0, int64_t nr, double* Bf, double* bmax,
                                                    const int32_t* gate) {
    if (gate && *gate == 0) return;
    __shared__ double red[256];
    const double inv_n = 1.0 / (double)*a.np;
    for (int64_t rl = blockIdx.x; rl < nr; rl += gridDim.x) {
        const int64_t r = r0 + rl;
        const int64_t srow = (int64_t)a.tsel[r / a.dy] * a.dy + r % a.dy;
        const double syv = a.sy[srow];
        double m = 0.0;
        const int64_t o = r % a.dy;
        for (int64_t i = threadIdx.x; i < a.d; i += 256) {
            const double v =
                cross_head(a.hdim, a.hper, o, i) ? 0.0 : (double)a.Syx[srow * a.d + i] - syv * a.sx[i] * inv_n;
            Bf[rl * a.d + i] = v;
            m = fmax(m, fabs(v));
        }
        if (!bmax) continue;
        red[threadIdx.x] = m;
        __syncthreads();
        for (int h = 128; h > 0; h >>= 1) {
            if ((int)threadIdx.x < h) red[threadIdx.x] = fmax(red[threadIdx.x], red[threadIdx.x + h]);
            __syncthreads();
        }
        if (threadIdx.x == 0) bmax[r] = red[0];
        __syncthreads();   // red is rewritten by the next row
    }
}

// The maps from the fp64 product, rows [r0, r0 + nr) (one row per work-group at a time, rows
// strided by the grid): W (fp32, may be null), the packed bf16 copy (may be null), and the
// intercept b = s_y / n - sum_j W[j] s_x[j] / n summed in fp64 in a fixed order (may be null).
__global__ __launch_bounds__(256) void k_store_f64(const double* Wf, int64_t r0, int64_t nr, CrossArgs a, float* W,
                                                   bf16_t* Wlp, float* b, const int32_t* gate) {
    if (gate && *gate == 0) return;
    __shared__ double red[256];
    const int64_t d = a.d;
    const double inv_n = 1.0 / (double)*a.np;
    for (int64_t rl = blockIdx.x; rl < nr; rl += gridDim.x) {
        const int64_t r = r0 + rl;
        const double* wr = Wf + rl * d;
        const int64_t wl_base = (r >> 8) * 256 * d + packed_row_part((int)(r & 255));
        double dot = 0.0;
        for (int64_t j = 4 * threadIdx.x; j < d; j += 1024) {
            const double w0 = wr[j], w1 = wr[j + 1], w2 = wr[j + 2], w3 = wr[j + 3];
            dot += w0 * a.sx[j] + w1 * a.sx[j + 1] + w2 * a.sx[j + 2] + w3 * a.sx[j + 3];
            // the bf16 map is the fp32 map rounded once more (not the double rounded once)
            const float f0 = opaque_f32((float)w0), f1 = opaque_f32((float)w1);
            const float f2 = opaque_f32((float)w2), f3 = opaque_f32((float)w3);
            if (W) *(f32x4*)(W + r * d + j) = f32x4{f0, f1, f2, f3};
            if (Wlp)
                *(u32x2*)(Wlp + wl_base + packed_col_part((int)j)) = u32x2{pack_bf16x2(f0, f1), pack_bf16x2(f2, f3)};
        }
        if (!b) continue;
        red[threadIdx.x] = dot;
        __syncthreads();
        for (int h = 128; h > 0; h >>= 1) {
            if ((int)threadIdx.x < h) red[threadIdx.x] += red[threadIdx.x + h];
            __syncthreads();
        }
        if (threadIdx.x == 0) {
            const int64_t srow = (int64_t)a.tsel[r / a.dy] * a.dy + r % a.dy;
            b[r] = (float)((a.sy[srow] - red[0]) * inv_n);
        }
        __syncthreads();   // red is rewritten by the next row
    }
}

// Wf[r - r0][j] = W[r][j] for rows [r0, r0 + nr) (fp32 maps widened for the residual product).
__global__ void k_widen_rows(const float* W, int64_t r0, int64_t nr, int64_t d, double* Wf) {
    const int64_t n = nr * d;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n; idx += (int64_t)gridDim.x * blockDim.x)
        Wf[idx] = (double)W[r0 * d + idx];
}

// rmax[r0 + row] = max_j |R[row][j]| (one work-group per row); NaN gives +inf.
__global__ __launch_bounds__(256) void k_row_absmax(const double* R, int64_t r0, int64_t d, double* rmax) {
    __shared__ double red[256];
    double m = 0.0;
    bool bad = false;
    for (int64_t j = threadIdx.x; j < d; j += 256) {
        const double v = R[(int64_t)blockIdx.x * d + j];
        m = fmax(m, fabs(v));
        bad |= v != v;
    }
    red[threadIdx.x] = bad ? INFINITY : m;
    __syncthreads();
    for (int h = 128; h > 0; h >>= 1) {
        if ((int)threadIdx.x < h) red[threadIdx.x] = fmax(red[threadIdx.x], red[threadIdx.x + h]);
        __syncthreads();
    }
    if (threadIdx.x == 0) rmax[r0 + blockIdx.x] = red[0];
}

// Per selected target i (one work-group each): max over its dy rows of the residual row maxima
// over the same for the centred cross moments.
__global__ __launch_bounds__(256) void k_resid_final(const double* rmax, const double* bmax, int64_t dy, double* out) {
    __shared__ double red[2][256];
    double mr = 0.0, mb = 0.0;
    for (int64_t o = threadIdx.x; o < dy; o += 256) {
        mr = fmax(mr, rmax[(int64_t)blockIdx.x * dy + o]);
        mb = fmax(mb, bmax[(int64_t)blockIdx.x * dy + o]);
    }
    red[0][threadIdx.x] = mr;
    red[1][threadIdx.x] = mb;
    __syncthreads();
    for (int h = 128; h > 0; h >>= 1) {
        if ((int)threadIdx.x < h) {
            red[0][threadIdx.x] = fmax(red[0][threadIdx.x], red[0][threadIdx.x + h]);
            red[1][threadIdx.x] = fmax(red[1][threadIdx.x], red[1][threadIdx.x + h]);
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) out[blockIdx.x] = red[0][0] / red[1][0];
}

// The route of one lambda: cond = the largest |entry| of the equilibrated inverse (from the
// tile maxima of k_split_inverse), gate = 1 when the fp64 product is to write the maps.
__global__ __launch_bounds__(256) void k_route(const double* hmax, int64_t n, int product, double cond_max,
                                               int32_t* gate, double* cond) {
    __shared__ double red[256];
    double m = 0.0;
    for (int64_t i = threadIdx.x; i < n; i += 256) m = fmax(m, hmax[i]);
    red[threadIdx.x] = m;
    __syncthreads();
    for (int h = 128; h > 0; h >>= 1) {
        if ((int)threadIdx.x < h) red[threadIdx.x] = fmax(red[threadIdx.x], red[threadIdx.x + h]);
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        const double c = red[0];
        if (cond) *cond = c;
        *gate = product == RF_PRODUCT_F64 || (product == RF_PRODUCT_AUTO && !(c <= cond_max));
    }
}

// -------------------------------------------------------------------------------------------
struct SolveWs {
    double *C, *Cinv, *Dinv, *mu_y, *dg, *rdg;   // C, Cinv, Dinv: one per lambda
    bf16_t *Aq, *Bq;
    float* bpart;
    double* hmax;      // per lambda: the tile maxima of the equilibrated inverse
    int32_t* gate;     // per lambda: 1 = the fp64 product writes the maps
    double *Bf, *Wf;   // fp64 row blocks of rb rows
    double *rmax, *bmax;
    int64_t rb;
    size_t total;
};

// Rows per fp64 block: 32 Mi elements of fp64 (256 MiB) per buffer, at least 64.  The fp64
// route's three launches per block run (and exit at once on their gate) whenever the route is
// automatic, so fewer, larger blocks keep that fixed cost small: at d = 4096 and 65536 rows,
// 8 blocks instead of 32 took about 0.1 ms less per solve (10.80-10.92 against 10.94-10.98 ms).
static int64_t f64_block_rows(int64_t d, int64_t rows) {
    int64_t rb = ((int64_t)(32 << 20) / d) / 64 * 64;
    if (rb < 64) rb = 64;
    return rows < rb ? rows : rb;
}

static SolveWs solve_ws(void* base, int64_t d, int64_t dy, int64_t n_sel, int64_t n_lam = 1) {
    SolveWs w{};
    size_t off = 0;
    char* p = (char*)base;
    auto take = [&](size_t bytes) {
        void* r = p ? (void*)(p + off) : nullptr;
        off += round_up(bytes, 256);
        return r;
    };
    const int64_t rows = n_sel * dy;
    w.C = (double*)take(n_lam * d * d * 8);
    w.Cinv = (double*)take(n_lam * d * d * 8);
    w.Dinv = (double*)take(n_lam * d * kNB * 8);
    w.mu_y = (double*)take(rows * 8);
    w.dg = (double*)take(d * 8);
    w.rdg = (double*)take(d * 8);
    w.Aq = (bf16_t*)take(rows * 2 * d * 2);
    w.Bq = (bf16_t*)take(d * 3 * d * 2);
    w.bpart = (float*)take(rows * (d / 256) * 4);
    w.hmax = (double*)take(n_lam * (d / 64) * (d / 64) * 8);
    w.gate = (int32_t*)take(n_lam * 4);
    w.rb = f64_block_rows(d, rows > 0 ? rows : 1);
    w.Bf = (double*)take(w.rb * d * 8);
    w.Wf = (double*)take(w.rb * d * 8);
    w.rmax = (double*)take((rows > 0 ? rows : 1) * 8);
    w.bmax = (double*)take((rows > 0 ? rows : 1) * 8);
    w.total = off;
    return w;
}

static inline unsigned grid_for(int64_t n, int64_t per = 256) {
    return (unsigned)std::max<int64_t>(1, std::min<int64_t>(ceil_div(n, per), 1 << 16));
}

// Work-groups of the row-strided fp64 route kernels: two per CU, few enough that a launch whose
// gate is off costs little.
constexpr unsigned kRowGrid = 512;
static inline unsigned row_grid(int64_t nr) { return (unsigned)std::max<int64_t>(1, std::min<int64_t>(nr, kRowGrid)); }

// 128 x 128 tiles only when they fill two rounds of the CUs at two work-groups each, else
// 64 x 64 tiles: more work-groups in flight at half the operand reuse (measured on the d=4096
// solve: 1024 tiles or more for 128 x 128 took 11.0 ms, 512 took 11.5 ms, and 128 x 128 tiles
// throughout the inverse 12.1 ms; 2048 and 64 x 64 throughout matched 1024)
constexpr int64_t kBigTiles = 1024;

// A batch of ``batch`` equal products sA, sB, sC elements apart (batch = 1: one product); the
// tile size is chosen from the tiles of the whole batch.  ``gate``: as for k_dgemm.
template <bool BT>
static rf_status dgemm(hipStream_t s, int64_t M, int64_t N, int64_t K, double alpha, const double* A, int64_t lda,
                       const double* B, int64_t ldb, double beta, double* C, int64_t ldc, int structure = kFull,
                       int batch = 1, int64_t sA = 0, int64_t sB = 0, int64_t sC = 0, const int32_t* gate = nullptr) {
    if (M <= 0 || N <= 0 || batch <= 0) return RF_OK;
    int64_t tiles = ceil_div(M, 128) * ceil_div(N, 128);
    if (structure & kLowerOnly) tiles = (tiles + ceil_div(M, 128)) / 2;
    tiles *= batch;
    if (tiles >= kBigTiles)
        hipLaunchKernelGGL((k_dgemm<BT, 128>), dim3((unsigned)ceil_div(M, 128), (unsigned)ceil_div(N, 128), (unsigned)batch),
                           dim3(256), 0, s, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, structure, sA, sB, sC, gate);
    else
        hipLaunchKernelGGL((k_dgemm<BT, 64>), dim3((unsigned)ceil_div(M, 64), (unsigned)ceil_div(N, 64), (unsigned)batch),
                           dim3(256), 0, s, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, structure, sA, sB, sC, gate);
    return check_launch("rf_solve: dgemm");
}

#define RF_TRY(expr)                      \
    do {                                  \
        rf_status _st = (expr);           \
        if (_st != RF_OK) return _st;     \
    } while (0)

// Z = L^-T = R^-1 with R = L^T upper triangular, by recursive doubling over unit size b =
// 64, 128, ...: at level b the rows split into units of b (the last one possibly shorter), and
// every pair of adjacent units (2p, 2p+1) is joined by
//   [[R11, R12], [0, R22]]^-1 = [[Z11, -Z11 R12 Z22], [0, Z22]],   R12 = L21^T,
// i.e. two products, T = Z11 L21^T and Z12 = -T Z22, batched over the pairs of whole units,
// with one more unbatched pair when the second unit of the last pair is short.  An unpaired
// last unit is carried to the next level unchanged.  Each unit is complete when it is used
// (by induction over the levels), and the number of dependent levels is log2(d / 64) rounded
// up, instead of one step per 64 columns.  The diagonal 64-blocks come from the factorisation
// (Dinv); T lives in the split-operand buffer, which is written only after the inverse.
// Lf holds the factor L (lower triangle), Dinv the inverses of its diagonal blocks.
static rf_status inverse_factor(hipStream_t s, const SolveWs& w, const double* Lf, const double* Dinv, int64_t d,
                                double* Z) {
    hipLaunchKernelGGL(k_zdiag, dim3(grid_for(d * d)), dim3(256), 0, s, Dinv, d, Z);
    RF_TRY(check_launch("rf_solve: inverse diagonal"));
    double* T = (double*)w.Bq;
    auto join = [&](int64_t o, int64_t b, int64_t n2, unsigned batch, int64_t sp) -> rf_status {
        // units [o, o + b) and [o + b, o + b + n2), repeated ``batch`` times every sp elements
        const bool big = ceil_div(b, 128) * ceil_div(n2, 128) * (int64_t)batch >= kBigTiles;
        const int64_t tb = big ? 128 : 64;
        const dim3 g1((unsigned)ceil_div(b, tb), (unsigned)ceil_div(n2, tb), batch);
        if (big)
            hipLaunchKernelGGL((k_dgemm<true, 128>), g1, dim3(256), 0, s, b, n2, b, 1.0, (const double*)(Z + o * d + o),
                               d, Lf + (o + b) * d + o, d, 0.0, T, n2, (int)kUpperA, sp, sp, b * n2,
                               (const int32_t*)nullptr);
        else
            hipLaunchKernelGGL((k_dgemm<true, 64>), g1, dim3(256), 0, s, b, n2, b, 1.0, (const double*)(Z + o * d + o),
                               d, Lf + (o + b) * d + o, d, 0.0, T, n2, (int)kUpperA, sp, sp, b * n2,
                               (const int32_t*)nullptr);
        RF_TRY(check_launch("rf_solve: inverse T"));
        if (big)
            hipLaunchKernelGGL((k_dgemm<false, 128>), g1, dim3(256), 0, s, b, n2, n2, -1.0, (const double*)T, n2,
                               (const double*)(Z + (o + b) * d + o + b), d, 0.0, Z + o * d + o + b, d, (int)kUpperB,
                               b * n2, sp, sp, (const int32_t*)nullptr);
        else
            hipLaunchKernelGGL((k_dgemm<false, 64>), g1, dim3(256), 0, s, b, n2, n2, -1.0, (const double*)T, n2,
                               (const double*)(Z + (o + b) * d + o + b), d, 0.0, Z + o * d + o + b, d, (int)kUpperB,
                               b * n2, sp, sp, (const int32_t*)nullptr);
        return check_launch("rf_solve: inverse Z12");
    };
    for (int64_t b = kNB; b < d; b *= 2) {
        const int64_t full = d / (2 * b);                 // pairs of whole units
        if (full > 0) RF_TRY(join(0, b, b, (unsigned)full, 2 * b * (d + 1)));
        const int64_t o = full * 2 * b;                   // a last pair with a short second unit
        if (o + b < d) RF_TRY(join(o, b, d - o - b, 1u, 0));
    }
    return RF_OK;
}

// The product stage for matrix z of the batch, whose inverse (or pseudo-inverse) stands in
// the lower triangle of w.C + z d^2 and whose split cross moments stand in w.Aq: the
// equilibrated split inverse and its largest entry (cond, may be null), the route, the split
// bf16 product (unless the route is fp64 only) and the fp64 product (unless it is split
// only; gated on the device under RF_PRODUCT_AUTO).  Writes W (fp32), W_lp (packed bf16) and
// b, each of which may be null.
static rf_status solve_products(hipStream_t s, const SolveWs& w, int z, int64_t d, int64_t rows, const CrossArgs& ca,
                                rf_product product, float* Wz, bf16_t* Wlpz, float* bz, double* cond) {
    const int64_t dd = d * d;
    const int64_t nb64 = (d / 64) * (d / 64);
    double* Cz = w.C + z * dd;
    int32_t* gz = w.gate + z;
    const double* sx = ca.sx;
    const int64_t* np = ca.np;
    // equilibrated split inverse (and its largest entry), then W on the MFMA pipes
    hipLaunchKernelGGL(k_split_inverse, dim3((unsigned)(d / 64), (unsigned)(d / 64)), dim3(256), 0, s, Cz, w.dg, d,
                       w.Bq, w.hmax + z * nb64);
    RF_TRY(check_launch("rf_solve: split inverse"));
    hipLaunchKernelGGL(k_route, dim3(1), dim3(256), 0, s, (const double*)(w.hmax + z * nb64), nb64, (int)product,
                       (double)RF_SPLIT_COND_MAX, gz, cond);
    RF_TRY(check_launch("rf_solve: route"));
    if (product != RF_PRODUCT_F64) {
        WArgs wa{};
        wa.Aq = w.Aq; wa.Bq = w.Bq; wa.rdg = w.rdg; wa.sx = sx; wa.np = np; wa.d = d; wa.rows = rows;
        wa.tiles_j = (int)(d / 256); wa.tiles_c = (int)(rows / 256); wa.W = Wz; wa.Wlp = Wlpz;
        wa.bpart = w.bpart;
        hipLaunchKernelGGL(k_wgemm, dim3((unsigned)(wa.tiles_j * wa.tiles_c)), dim3(PackedAGemm::kThr), 0, s, wa);
        RF_TRY(check_launch("rf_solve: W product"));
        if (bz) {
            hipLaunchKernelGGL(k_bias, dim3((unsigned)ceil_div(rows, 256)), dim3(256), 0, s, w.bpart, wa.tiles_j,
                               w.mu_y, rows, bz);
            RF_TRY(check_launch("rf_solve: bias"));
        }
    }
    if (product != RF_PRODUCT_SPLIT_BF16) {
        // the fp64 product, written over the split one when the route says so:
        // W = B A^-1 with the full A^-1 (mirrored into the free Z buffer), rb rows at a time
        double* Af = w.Cinv + z * dd;
        hipLaunchKernelGGL(k_mirror_full, dim3(std::min(grid_for(dd), kRowGrid * 4)), dim3(256), 0, s,
                           (const double*)Cz, d, Af, (const int32_t*)gz);
        RF_TRY(check_launch("rf_solve: fp64 inverse"));
        for (int64_t r0 = 0; r0 < rows; r0 += w.rb) {
            const int64_t nr = std::min<int64_t>(w.rb, rows - r0);
            hipLaunchKernelGGL(k_centre_f64, dim3(row_grid(nr)), dim3(256), 0, s, ca, r0, nr, w.Bf,
                               (double*)nullptr, (const int32_t*)gz);
            RF_TRY(check_launch("rf_solve: fp64 cross moments"));
            RF_TRY(dgemm<false>(s, nr, d, d, 1.0, w.Bf, d, Af, d, 0.0, w.Wf, d, kFull, 1, 0, 0, 0, gz));
            hipLaunchKernelGGL(k_store_f64, dim3(row_grid(nr)), dim3(256), 0, s, (const double*)w.Wf, r0, nr, ca, Wz,
                               Wlpz, bz, (const int32_t*)gz);
            RF_TRY(check_launch("rf_solve: fp64 maps"));
        }
    }
    return RF_OK;
}

// ---- eigendecomposition route (pseudo-inverse) ---------------------------------------------
// Cyclic Jacobi in round-robin order: in round r of a sweep the d players (indices) meet in
// d/2 disjoint pairs (player 0 fixed, the others turning one seat per round), so every pair
// meets once per sweep and a round's rotations commute.

// The player in seat ``pos`` of round r.
__device__ inline int64_t rr_player(int64_t pos, int64_t r, int64_t d) {
    return pos == 0 ? 0 : 1 + ((pos - 1 - r) % (d - 1) + (d - 1)) % (d - 1);
}

// Pair k of round r: (p, q) = the players in seats k and d-1-k, p < q, and the rotation (c, s)
// that zeroes A[p][q] in J^T A J with J = I except J_pp = J_qq = c, J_pq = s, J_qp = -s
// (the symmetric 2 x 2 Schur step).  A pair already below fp64 resolution keeps (1, 0).
__global__ void k_jacobi_angles(const double* A, int64_t d, int64_t r, double* cs, int64_t* pq) {
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= d / 2) return;
    int64_t p = rr_player(k, r, d), q = rr_player(d - 1 - k, r, d);
    if (p > q) {
        const int64_t t = p;
        p = q;
        q = t;
    }
    const double app = A[p * d + p], aqq = A[q * d + q], apq = A[p * d + q];
    double c = 1.0, s = 0.0;
    if (apq != 0.0 && fabs(apq) > 1e-300 + 1e-18 * sqrt(fabs(app * aqq))) {
        const double tau = (aqq - app) / (2.0 * apq);
        const double t = (tau >= 0.0 ? 1.0 : -1.0) / (fabs(tau) + sqrt(tau * tau + 1.0));
        c = 1.0 / sqrt(t * t + 1.0);
        s = t * c;
    }
    cs[2 * k] = c;
    cs[2 * k + 1] = s;
    pq[2 * k] = p;
    pq[2 * k + 1] = q;
}

// A <- J^T A J and V <- V J for all pairs of the round: each 2 x 2 block (pair i rows, pair j
// columns) of A changes on its own, as does each (row, pair j) couple of V.
__global__ void k_jacobi_rotate(double* A, double* V, int64_t d, const double* cs, const int64_t* pq) {
    const int64_t h = d / 2;
    const int64_t na = h * h, nv = d * h;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < na + nv;
         t += (int64_t)gridDim.x * blockDim.x) {
        if (t < na) {
            const int64_t i = t / h, j = t - i * h;
            const int64_t p = pq[2 * i], q = pq[2 * i + 1], u = pq[2 * j], w = pq[2 * j + 1];
            const double ci = cs[2 * i], si = cs[2 * i + 1], cj = cs[2 * j], sj = cs[2 * j + 1];
            const double a00 = A[p * d + u], a01 = A[p * d + w], a10 = A[q * d + u], a11 = A[q * d + w];
            // rows: p' = c p - s q, q' = s p + c q; then columns the same way with pair j's turn
            const double r00 = ci * a00 - si * a10, r01 = ci * a01 - si * a11;
            const double r10 = si * a00 + ci * a10, r11 = si * a01 + ci * a11;
            A[p * d + u] = cj * r00 - sj * r01;
            A[p * d + w] = sj * r00 + cj * r01;
            A[q * d + u] = cj * r10 - sj * r11;
            A[q * d + w] = sj * r10 + cj * r11;
        } else {
            const int64_t e = t - na;
            const int64_t row = e / h, j = e - row * h;
            const int64_t u = pq[2 * j], w = pq[2 * j + 1];
            const double cj = cs[2 * j], sj = cs[2 * j + 1];
            const double v0 = V[row * d + u], v1 = V[row * d + w];
            V[row * d + u] = cj * v0 - sj * v1;
            V[row * d + w] = sj * v0 + cj * v1;
        }
    }
}

__global__ void k_identity(double* V, int64_t d) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < d * d; i += (int64_t)gridDim.x * blockDim.x)
        V[i] = (i / d == i % d) ? 1.0 : 0.0;
}

// U = V diag(sqrt(f)) with f_i = 1/mu_i for mu_i = A[i][i] > rel_tol * max mu, else 0, so that
// U U^T is the pseudo-inverse.  One work-group finds the largest eigenvalue; the scaling is
// grid-strided over the elements of V (every work-group recomputes the maximum).
__global__ __launch_bounds__(256) void k_pinv_scale(const double* A, int64_t d, double rel_tol, double* V) {
    __shared__ double red[256];
    double m = -INFINITY;
    for (int64_t i = threadIdx.x; i < d; i += 256) m = fmax(m, A[i * d + i]);
    red[threadIdx.x] = m;
    __syncthreads();
    for (int h = 128; h > 0; h >>= 1) {
        if ((int)threadIdx.x < h) red[threadIdx.x] = fmax(red[threadIdx.x], red[threadIdx.x + h]);
        __syncthreads();
    }
    const double cut = rel_tol * red[0];
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < d * d; e += (int64_t)gridDim.x * blockDim.x) {
        const int64_t col = e % d;
        const double mu = A[col * d + col];
        V[e] = (red[0] > 0.0 && mu > cut) ? V[e] / sqrt(mu) : 0.0;
    }
}

// All rows of the centred, equilibrated, split cross moments (the Cholesky route computes them
// in the spare work-groups of its diagonal-block launches).
__global__ __launch_bounds__(256) void k_centre_split(CrossArgs ca, int ny) {
    const int64_t c = blockIdx.x / ny;
    const int64_t i0 = ((blockIdx.x % ny) * 256 + threadIdx.x) * 8;
    if (c < ca.rows && i0 < ca.d) centre_split_row(ca, c, i0);
}

// ---- fit quality ------------------------------------------------------------------------
constexpr int kR2Rows = 16;   // map rows per work-group

// Per (target, block of kR2Rows rows): fp64 partial sums of W[o][i] * B[o][i] and W[o][i]^2 with
// B = S_yx - s_y s_x^T / n, each thread over a fixed set of elements, then a fixed-order tree.
__global__ __launch_bounds__(256) void k_r2_partial(const float* Syx, const double* sy, const double* sx,
                                                     const int64_t* np, const float* W, int64_t d, int64_t dy,
                                                     CrossArgs ca, int n_blk, double* part) {
    const int l = blockIdx.y, blk = blockIdx.x;
    const double inv_n = 1.0 / (double)*np;
    double dot = 0.0, ww = 0.0;
    for (int r = 0; r < kR2Rows; ++r) {
        const int64_t o = (int64_t)blk * kR2Rows + r;
        if (o >= dy) break;
        const int64_t srow = (int64_t)ca.tsel[l] * dy + o;
        const float* wrow = W + ((int64_t)l * dy + o) * d;
        const float* brow = Syx + srow * d;
        const double syv = sy[srow] * inv_n;
        for (int64_t i = threadIdx.x * 4; i < d; i += 1024) {
            const f32x4 w = *(const f32x4*)(wrow + i);
            const f32x4 b = *(const f32x4*)(brow + i);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const double wd = (double)w[e];
                dot += wd * ((double)b[e] - syv * sx[i + e]);
                ww += wd * wd;
            }
        }
    }
    __shared__ double red[2][256];
    red[0][threadIdx.x] = dot;
    red[1][threadIdx.x] = ww;
    __syncthreads();
    for (int h = 128; h > 0; h >>= 1) {
        if ((int)threadIdx.x < h) {
            red[0][threadIdx.x] += red[0][threadIdx.x + h];
            red[1][threadIdx.x] += red[1][threadIdx.x + h];
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        part[((int64_t)l * n_blk + blk) * 2] = red[0][0];
        part[((int64_t)l * n_blk + blk) * 2 + 1] = red[1][0];
    }
}

// One work-group per target: the partials in block order, SST from the column sums, the
// absolute ridge strength, and R^2.
__global__ __launch_bounds__(256) void k_r2_final(const float* Sxx, const double* sx, const double* sy,
                                                   const double* syy, const int64_t* np, int64_t d, int64_t dy,
                                                   CrossArgs ca, int n_blk, const double* part, double lambda,
                                                   int rel, double* r2) {
    const int l = blockIdx.x;
    const double n = (double)*np;
    __shared__ double red[3][256];
    double sst = 0.0, diag = 0.0;
    for (int64_t o = threadIdx.x; o < dy; o += 256) {
        const int64_t srow = (int64_t)ca.tsel[l] * dy + o;
        sst += syy[srow] - sy[srow] * sy[srow] / n;
    }
    if (rel)
        for (int64_t i = threadIdx.x; i < d; i += 256) diag += (double)Sxx[i * d + i] - sx[i] * sx[i] / n;
    red[0][threadIdx.x] = sst;
    red[1][threadIdx.x] = diag;
    __syncthreads();
    for (int h = 128; h > 0; h >>= 1) {
        if ((int)threadIdx.x < h) {
            red[0][threadIdx.x] += red[0][threadIdx.x + h];
            red[1][threadIdx.x] += red[1][threadIdx.x + h];
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        double dot = 0.0, ww = 0.0;
        for (int b = 0; b < n_blk; ++b) {
            dot += part[((int64_t)l * n_blk + b) * 2];
            ww += part[((int64_t)l * n_blk + b) * 2 + 1];
        }
        const double lam = rel ? lambda * red[1][0] / (double)d : lambda;
        r2[l] = (dot + lam * ww) / red[0][0];
    }
}

}  // namespace rf

using namespace rf;

extern "C" {

size_t rf_fit_r2_workspace_bytes(const rf_gram_desc* desc, int32_t n_sel) {
    rf_gram_layout_t GL;
    if (n_sel < 0 || rf_gram_state_layout(desc, &GL) != RF_OK) return 0;
    return round_up((size_t)n_sel * (size_t)ceil_div(gram_dy(desc), kR2Rows) * 2 * sizeof(double), 256);
}

rf_status rf_fit_r2(const rf_gram_desc* desc, const void* d_state, double lambda, rf_lambda_mode mode,
                    const int32_t* targets, int32_t n_sel, const float* d_W, double* d_r2, void* d_ws,
                    size_t ws_bytes, void* stream) {
    clear_error();
    rf_gram_layout_t GL;
    rf_status st = rf_gram_state_layout(desc, &GL);
    if (st != RF_OK) return st;
    RF_REQUIRE(d_state && aligned(d_state, 256), RF_ERR_INVALID_ARG, "rf_fit_r2: state must be non-null, 256-B aligned");
    RF_REQUIRE(isfinite(lambda) && lambda >= 0.0, RF_ERR_INVALID_ARG, "rf_fit_r2: lambda must be finite and >= 0");
    RF_REQUIRE(mode == RF_LAMBDA_ABSOLUTE || mode == RF_LAMBDA_REL_MEAN_DIAG, RF_ERR_INVALID_ARG,
               "rf_fit_r2: bad lambda mode");
    RF_REQUIRE(n_sel >= 0 && n_sel <= kMaxSel, RF_ERR_UNSUPPORTED, "rf_fit_r2: 0..64 selected targets");
    if (n_sel == 0) return RF_OK;
    RF_REQUIRE(targets && d_W && d_r2, RF_ERR_INVALID_ARG, "rf_fit_r2: null pointer argument");
    for (int i = 0; i < n_sel; ++i)
        RF_REQUIRE(targets[i] >= 0 && targets[i] < desc->n_targets, RF_ERR_INVALID_ARG,
                   "rf_fit_r2: target index out of range");
    RF_REQUIRE(aligned(d_W, 16) && aligned(d_r2, 8), RF_ERR_INVALID_ARG, "rf_fit_r2: W must be 16-byte aligned");
    RF_REQUIRE(d_ws && aligned(d_ws, 256), RF_ERR_INVALID_ARG, "rf_fit_r2: workspace must be non-null, 256-B aligned");
    RF_REQUIRE(ws_bytes >= rf_fit_r2_workspace_bytes(desc, n_sel), RF_ERR_WORKSPACE, "rf_fit_r2: workspace too small");
    const int64_t d = desc->d, dy = gram_dy(desc);
    const char* sp = (const char*)d_state;
    CrossArgs ca{};
    for (int i = 0; i < n_sel; ++i) ca.tsel[i] = targets[i];
    const int n_blk = (int)ceil_div(dy, kR2Rows);
    hipStream_t s = (hipStream_t)stream;
    hipLaunchKernelGGL(k_r2_partial, dim3((unsigned)n_blk, (unsigned)n_sel), dim3(256), 0, s,
                       (const float*)(sp + GL.off_S_yx), (const double*)(sp + GL.off_s_y),
                       (const double*)(sp + GL.off_s_x), (const int64_t*)(sp + GL.off_n), d_W, d, dy, ca, n_blk,
                       (double*)d_ws);
    RF_TRY(check_launch("rf_fit_r2: partial sums"));
    hipLaunchKernelGGL(k_r2_final, dim3((unsigned)n_sel), dim3(256), 0, s, (const float*)(sp + GL.off_S_xx),
                       (const double*)(sp + GL.off_s_x), (const double*)(sp + GL.off_s_y),
                       (const double*)(sp + GL.off_s_yy), (const int64_t*)(sp + GL.off_n), d, dy, ca, n_blk,
                       (const double*)d_ws, lambda, (int)(mode == RF_LAMBDA_REL_MEAN_DIAG), d_r2);
    return check_launch("rf_fit_r2: scores");
}

static size_t pinv_extra_bytes(int64_t d) { return round_up((size_t)(d * d * 8), 256) + round_up((size_t)d * 16, 256) * 2; }

size_t rf_solve_pinv_workspace_bytes(const rf_gram_desc* desc, int32_t n_sel) {
    rf_gram_layout_t GL;
    if (n_sel < 0 || rf_gram_state_layout(desc, &GL) != RF_OK) return 0;
    return solve_ws(nullptr, desc->d, gram_dy(desc), n_sel, 1).total + pinv_extra_bytes(desc->d);
}

rf_status rf_solve_pinv(const rf_gram_desc* desc, const void* d_state, double lambda, rf_lambda_mode mode,
                        double rel_tol, int32_t sweeps, const int32_t* targets, int32_t n_sel, float* d_W,
                        void* d_W_lp, float* d_b, void* d_ws, size_t ws_bytes, void* stream) {
    clear_error();
    rf_gram_layout_t GL;
    rf_status st = rf_gram_state_layout(desc, &GL);
    if (st != RF_OK) return st;
    RF_REQUIRE(d_state && aligned(d_state, 256), RF_ERR_INVALID_ARG, "rf_solve_pinv: state must be non-null, 256-B aligned");
    RF_REQUIRE(isfinite(lambda) && lambda >= 0.0, RF_ERR_INVALID_ARG, "rf_solve_pinv: lambda must be finite and >= 0");
    RF_REQUIRE(mode == RF_LAMBDA_ABSOLUTE || mode == RF_LAMBDA_REL_MEAN_DIAG, RF_ERR_INVALID_ARG,
               "rf_solve_pinv: bad lambda mode");
    RF_REQUIRE(isfinite(rel_tol) && rel_tol >= 0.0 && rel_tol < 1.0, RF_ERR_INVALID_ARG,
               "rf_solve_pinv: rel_tol must be in [0, 1)");
    RF_REQUIRE(sweeps >= 1 && sweeps <= 64, RF_ERR_INVALID_ARG, "rf_solve_pinv: sweeps must be in [1, 64]");
    RF_REQUIRE(n_sel >= 0 && n_sel <= kMaxSel, RF_ERR_UNSUPPORTED, "rf_solve_pinv: 0..64 selected targets");
    RF_REQUIRE(n_sel == 0 || targets, RF_ERR_INVALID_ARG, "rf_solve_pinv: null targets");
    for (int i = 0; i < n_sel; ++i)
        RF_REQUIRE(targets[i] >= 0 && targets[i] < desc->n_targets, RF_ERR_INVALID_ARG,
                   "rf_solve_pinv: target index out of range");
    RF_REQUIRE(aligned(d_ws, 256), RF_ERR_INVALID_ARG, "rf_solve_pinv: workspace must be 256-B aligned");
    RF_REQUIRE(aligned(d_W, 16) && aligned(d_W_lp, 16) && aligned(d_b, 4), RF_ERR_INVALID_ARG,
               "rf_solve_pinv: W outputs must be 16-byte aligned");
    const int64_t d = desc->d, dy = gram_dy(desc);
    const SolveWs w = solve_ws(d_ws, d, dy, n_sel, 1);
    RF_REQUIRE(d_ws && ws_bytes >= w.total + pinv_extra_bytes(d), RF_ERR_WORKSPACE, "rf_solve_pinv: workspace too small");
    double* V = (double*)((char*)d_ws + w.total);
    double* cs = (double*)((char*)V + round_up((size_t)(d * d * 8), 256));
    int64_t* pq = (int64_t*)((char*)cs + round_up((size_t)d * 16, 256));
    hipStream_t s = (hipStream_t)stream;
    const char* sp = (const char*)d_state;
    const float* Sxx = (const float*)(sp + GL.off_S_xx);
    const double* sx = (const double*)(sp + GL.off_s_x);
    const int64_t* np = (const int64_t*)(sp + GL.off_n);

    hipLaunchKernelGGL(k_centre_gram, dim3(grid_for(d * d)), dim3(256), 0, s, Sxx, sx, np, d, w.C, 0, 0);
    RF_TRY(check_launch("rf_solve_pinv: centre"));
    Lambdas lams{};
    lams.v[0] = lambda;
    hipLaunchKernelGGL(k_add_lambda, dim3(1), dim3(256), 0, s, w.C, d, lams, (int)(mode == RF_LAMBDA_REL_MEAN_DIAG));
    RF_TRY(check_launch("rf_solve_pinv: lambda"));
    hipLaunchKernelGGL(k_diag_sqrt, dim3(grid_for(d)), dim3(256), 0, s, w.C, d, w.dg, w.rdg);
    RF_TRY(check_launch("rf_solve_pinv: diagonal"));
    // A = V diag(mu) V^T by cyclic Jacobi (A becomes diag(mu) in place)
    hipLaunchKernelGGL(k_identity, dim3(grid_for(d * d)), dim3(256), 0, s, V, d);
    RF_TRY(check_launch("rf_solve_pinv: identity"));
    const int64_t n_rot = (d / 2) * (d / 2) + d * (d / 2);
    for (int sw = 0; sw < sweeps; ++sw) {
        for (int64_t r = 0; r < d - 1; ++r) {
            hipLaunchKernelGGL(k_jacobi_angles, dim3((unsigned)ceil_div(d / 2, 256)), dim3(256), 0, s, (const double*)w.C,
                               d, r, cs, pq);
            hipLaunchKernelGGL(k_jacobi_rotate, dim3(grid_for(n_rot)), dim3(256), 0, s, w.C, V, d, (const double*)cs,
                               (const int64_t*)pq);
        }
        RF_TRY(check_launch("rf_solve_pinv: Jacobi sweep"));
    }
    // U = V diag(1/sqrt(mu)) over the kept eigenvalues; A^+ = U U^T (lower triangle, as the W
    // product's operand preparation reads it)
    hipLaunchKernelGGL(k_pinv_scale, dim3(grid_for(d * d)), dim3(256), 0, s, (const double*)w.C, d, rel_tol, V);
    RF_TRY(check_launch("rf_solve_pinv: scale"));
    RF_TRY(dgemm<true>(s, d, d, d, 1.0, V, d, V, d, 0.0, w.C, d, kLowerOnly));
    if (n_sel == 0) return RF_OK;
    const int64_t rows = (int64_t)n_sel * dy;
    CrossArgs ca{};
    ca.Syx = (const float*)(sp + GL.off_S_yx); ca.sy = (const double*)(sp + GL.off_s_y); ca.sx = sx; ca.np = np;
    ca.rdg = w.rdg; ca.d = d; ca.dy = dy; ca.rows = rows; ca.Aq = w.Aq; ca.mu_y = w.mu_y;
    for (int i = 0; i < n_sel; ++i) ca.tsel[i] = targets[i];
    const int ny = (int)ceil_div(d, 2048);
    hipLaunchKernelGGL(k_centre_split, dim3((unsigned)(rows * ny)), dim3(256), 0, s, ca, ny);
    RF_TRY(check_launch("rf_solve_pinv: cross moments"));
    // the maps from the pseudo-inverse: the split product, or the fp64 one where the
    // equilibrated pseudo-inverse is too large for it (as rf_solve's RF_PRODUCT_AUTO)
    RF_TRY(solve_products(s, w, 0, d, rows, ca, RF_PRODUCT_AUTO, d_W, (bf16_t*)d_W_lp, d_b, nullptr));
    return RF_OK;
}

size_t rf_solve_workspace_bytes(const rf_gram_desc* desc, int32_t n_sel, int32_t n_lambda) {
    rf_gram_layout_t GL;
    if (n_sel < 0 || n_lambda < 1 || n_lambda > kMaxLambda || rf_gram_state_layout(desc, &GL) != RF_OK) return 0;
    return solve_ws(nullptr, desc->d, gram_dy(desc), n_sel, n_lambda).total;
}

rf_status rf_info_status(const int32_t* info, int32_t n) {
    clear_error();
    RF_REQUIRE(n >= 0 && (n == 0 || info), RF_ERR_INVALID_ARG, "rf_info_status: null info");
    for (int32_t i = 0; i < n; ++i)
        if (info[i] != 0)
            return fail(RF_ERR_NOT_SPD, "lambda " + std::to_string(i) + ": the regularised Gram is not positive definite "
                                        "(first failing leading minor " + std::to_string(info[i]) + ")");
    return RF_OK;
}

}  // extern "C"

namespace rf {
// rf_solve, and rf_solve_headwise with hdim = the head width (0: dense maps).
static rf_status solve_impl(const rf_gram_desc* desc, const void* d_state, const double* lambdas, int32_t n_lambda,
                            rf_lambda_mode mode, const int32_t* targets, int32_t n_sel, rf_product product,
                            float* d_W, void* d_W_lp, float* d_b, int32_t* d_info, double* d_cond, double* d_resid,
                            void* d_ws, size_t ws_bytes, void* stream, int32_t hdim) {
    rf_gram_layout_t GL;
    rf_status st = rf_gram_state_layout(desc, &GL);
    if (st != RF_OK) return st;
    RF_REQUIRE(d_state && aligned(d_state, 256), RF_ERR_INVALID_ARG, "rf_solve: state must be non-null, 256-B aligned");
    RF_REQUIRE(d_info, RF_ERR_INVALID_ARG, "rf_solve: null info");
    RF_REQUIRE(lambdas && n_lambda >= 1 && n_lambda <= kMaxLambda, RF_ERR_INVALID_ARG,
               "rf_solve: need 1..8 lambdas (host array)");
    for (int i = 0; i < n_lambda; ++i)
        RF_REQUIRE(isfinite(lambdas[i]) && lambdas[i] >= 0.0, RF_ERR_INVALID_ARG, "rf_solve: lambda must be finite and >= 0");
    RF_REQUIRE(mode == RF_LAMBDA_ABSOLUTE || mode == RF_LAMBDA_REL_MEAN_DIAG, RF_ERR_INVALID_ARG, "rf_solve: bad lambda mode");
    RF_REQUIRE(product == RF_PRODUCT_AUTO || product == RF_PRODUCT_SPLIT_BF16 || product == RF_PRODUCT_F64,
               RF_ERR_INVALID_ARG, "rf_solve: bad product route");
    RF_REQUIRE(n_sel >= 0 && n_sel <= kMaxSel, RF_ERR_UNSUPPORTED, "rf_solve: 0..64 selected targets");
    RF_REQUIRE(n_sel == 0 || targets, RF_ERR_INVALID_ARG, "rf_solve: null targets");
    for (int i = 0; i < n_sel; ++i)
        RF_REQUIRE(targets[i] >= 0 && targets[i] < desc->n_targets, RF_ERR_INVALID_ARG, "rf_solve: target index out of range");
    RF_REQUIRE(aligned(d_ws, 256), RF_ERR_INVALID_ARG, "rf_solve: workspace must be 256-B aligned");
    RF_REQUIRE(aligned(d_W, 16) && aligned(d_W_lp, 16) && aligned(d_b, 4) && aligned(d_cond, 8) && aligned(d_resid, 8),
               RF_ERR_INVALID_ARG, "rf_solve: W outputs must be 16-byte aligned");
    RF_REQUIRE(!d_resid || d_W, RF_ERR_INVALID_ARG, "rf_solve: the residual is computed from the fp32 maps (d_W)");
    const int64_t d = desc->d, dy = gram_dy(desc);
    const int nl = n_lambda;
    const SolveWs w = solve_ws(d_ws, d, dy, n_sel, nl);
    RF_REQUIRE(d_ws && ws_bytes >= w.total, RF_ERR_WORKSPACE, "rf_solve: workspace too small");
    hipStream_t s = (hipStream_t)stream;
    const char* sp = (const char*)d_state;
    const float* Sxx = (const float*)(sp + GL.off_S_xx);
    const float* Syx = (const float*)(sp + GL.off_S_yx);
    const double* sx = (const double*)(sp + GL.off_s_x);
    const double* sy = (const double*)(sp + GL.off_s_y);
    const int64_t* np = (const int64_t*)(sp + GL.off_n);
    const int64_t dd = d * d;
    const int rel = (int)(mode == RF_LAMBDA_REL_MEAN_DIAG);
    Lambdas lams{};
    for (int i = 0; i < nl; ++i) lams.v[i] = lambdas[i];

    // A_z = C + lambda_z I for every lambda of the batch; the equilibration D = diag(A_0) is
    // shared by the batch (any positive diagonal scaling leaves the products exact in theory;
    // one D lets the split cross moments serve every lambda)
    hipLaunchKernelGGL(k_zero_int, dim3(1), dim3(64), 0, s, d_info, nl);
    RF_TRY(check_launch("rf_solve: info"));
    const int32_t hper = (int32_t)dy;
    hipLaunchKernelGGL(k_centre_gram, dim3(grid_for(dd), (unsigned)nl), dim3(256), 0, s, Sxx, sx, np, d, w.C, hdim,
                       hper);
    RF_TRY(check_launch("rf_solve: centre"));
    hipLaunchKernelGGL(k_add_lambda, dim3((unsigned)nl), dim3(256), 0, s, w.C, d, lams, rel);
    RF_TRY(check_launch("rf_solve: lambda"));
    hipLaunchKernelGGL(k_diag_sqrt, dim3(grid_for(d)), dim3(256), 0, s, w.C, d, w.dg, w.rdg);
    RF_TRY(check_launch("rf_solve: diagonal"));

    // centred, equilibrated, split cross moments: computed in slices by the diagonal-block
    // launches' spare work-groups
    const int64_t rows = (int64_t)n_sel * dy;
    CrossArgs ca{};
    ca.Syx = Syx; ca.sy = sy; ca.sx = sx; ca.np = np; ca.rdg = w.rdg; ca.d = d; ca.dy = dy; ca.rows = rows; ca.Aq = w.Aq;
    ca.mu_y = w.mu_y; ca.hdim = hdim; ca.hper = hper;
    for (int i = 0; i < n_sel; ++i) ca.tsel[i] = targets[i];
    const int ny = (int)ceil_div(d, 2048);

    // blocked Cholesky of every A_z (batched over the lambdas): step J factors diagonal block J,
    // solves its panel, updates block column J + 1, then factors diagonal block J + 1 in the same
    // launch as the rest of step J's trailing update, so the diagonal factorisations (one wave
    // each, a serial chain) run beside the trailing updates instead of between them
    const int nblk = (int)(d / kNB);
    const int64_t rows_per = ceil_div(rows, nblk);
    auto slice = [&](int J, int64_t& cb, int64_t& ce) {
        cb = std::min<int64_t>(rows, J * rows_per);
        ce = std::min<int64_t>(rows, cb + rows_per);
    };
    {
        int64_t cb, ce;
        slice(0, cb, ce);
        hipLaunchKernelGGL(k_chol_diag, dim3((unsigned)(nl + (ce - cb) * ny)), dim3(256), 0, s, w.C, dd, d, 0, w.Dinv,
                           d * kNB, d_info, nl, ca, cb, ce, ny);
        RF_TRY(check_launch("rf_solve: potrf"));
    }
    for (int J = 0; J + 1 < nblk; ++J) {
        const int64_t c0 = (int64_t)J * kNB;
        const int64_t rem = d - c0 - kNB;
        // L21 = A21 L11^-T in place on the matrix cores: one column of 64 x 64 tiles, each of which
        // reads all of its rows of A21 before writing them
        double* panel = w.C + (c0 + kNB) * d + c0;
        hipLaunchKernelGGL((k_dgemm<true, 64>), dim3((unsigned)ceil_div(rem, 64), 1u, (unsigned)nl), dim3(256), 0, s,
                           rem, (int64_t)kNB, (int64_t)kNB, 1.0, (const double*)panel, d,
                           (const double*)(w.Dinv + c0 * kNB), (int64_t)kNB, 0.0, panel, d, (int)kFull, dd, d * kNB, dd,
                           (const int32_t*)nullptr);
        RF_TRY(check_launch("rf_solve: panel"));
        // block column J + 1 of the trailing update (all rows below block J)
        RF_TRY(dgemm<true>(s, rem, kNB, kNB, -1.0, panel, d, panel, d, 1.0, w.C + (c0 + kNB) * d + c0 + kNB, d, kFull,
                           nl, dd, dd, dd));
        // diagonal block J + 1 beside the rest of the update (rows and columns past block J + 1)
        const int64_t m = rem - kNB, tm = ceil_div(m, 64);
        const TrailArgs u{panel + kNB * d, w.C + (c0 + 2 * kNB) * d + c0 + 2 * kNB, m, m > 0 ? tm * (tm + 1) / 2 : 0};
        int64_t cb, ce;
        slice(J + 1, cb, ce);
        hipLaunchKernelGGL(k_chol_step, dim3((unsigned)(nl + u.tiles * nl + (ce - cb) * ny)), dim3(256), 0, s, w.C, dd,
                           d, J + 1, w.Dinv, d * kNB, d_info, nl, u, ca, cb, ce, ny);
        RF_TRY(check_launch("rf_solve: potrf step"));
    }
    for (int z = 0; z < nl; ++z) {
        double* Cz = w.C + z * dd;
        double* Zz = w.Cinv + z * dd;
        // A^-1 = Z Z^T with Z = L^-T (the factor is no longer needed afterwards: A^-1 overwrites it)
        RF_TRY(inverse_factor(s, w, Cz, w.Dinv + z * d * kNB, d, Zz));
        // lower triangle only (by 128-blocks): A^-1 is symmetric and its readers mirror it
        RF_TRY(dgemm<true>(s, d, d, d, 1.0, Zz, d, Zz, d, 0.0, Cz, d, kUpperOperands | kLowerOnly));
    }
    if (n_sel == 0) return RF_OK;

    for (int z = 0; z < nl; ++z) {
        float* Wz = d_W ? d_W + z * rows * d : nullptr;
        bf16_t* Wlpz = d_W_lp ? (bf16_t*)d_W_lp + z * rows * d : nullptr;
        float* bz = d_b ? d_b + z * rows : nullptr;
        RF_TRY(solve_products(s, w, z, d, rows, ca, product, Wz, Wlpz, bz, d_cond ? d_cond + z : nullptr));
        if (d_resid) {
            // stationarity residual in fp64: R = W A - B with A rebuilt from the state
            double* Af = w.Cinv + z * dd;
            hipLaunchKernelGGL(k_centre_gram, dim3(grid_for(dd), 1u), dim3(256), 0, s, Sxx, sx, np, d, Af, hdim, hper);
            RF_TRY(check_launch("rf_solve: residual matrix"));
            Lambdas one{};
            one.v[0] = lambdas[z];
            hipLaunchKernelGGL(k_add_lambda, dim3(1), dim3(256), 0, s, Af, d, one, rel);
            RF_TRY(check_launch("rf_solve: residual lambda"));
            for (int64_t r0 = 0; r0 < rows; r0 += w.rb) {
                const int64_t nr = std::min<int64_t>(w.rb, rows - r0);
                hipLaunchKernelGGL(k_centre_f64, dim3(row_grid(nr)), dim3(256), 0, s, ca, r0, nr, w.Bf, w.bmax,
                                   (const int32_t*)nullptr);
                RF_TRY(check_launch("rf_solve: residual cross moments"));
                hipLaunchKernelGGL(k_widen_rows, dim3(grid_for(nr * d)), dim3(256), 0, s, (const float*)Wz, r0, nr, d,
                                   w.Wf);
                RF_TRY(check_launch("rf_solve: residual maps"));
                RF_TRY(dgemm<false>(s, nr, d, d, 1.0, w.Wf, d, Af, d, -1.0, w.Bf, d));
                hipLaunchKernelGGL(k_row_absmax, dim3((unsigned)nr), dim3(256), 0, s, (const double*)w.Bf, r0, d, w.rmax);
                RF_TRY(check_launch("rf_solve: residual maxima"));
            }
            hipLaunchKernelGGL(k_resid_final, dim3((unsigned)n_sel), dim3(256), 0, s, (const double*)w.rmax,
                               (const double*)w.bmax, dy, d_resid + (int64_t)z * n_sel);
            RF_TRY(check_launch("rf_solve: residual"));
        }
    }
    return RF_OK;
}
}  // namespace rf

extern "C" {

rf_status rf_solve(const rf_gram_desc* desc, const void* d_state, const double* lambdas, int32_t n_lambda,
                   rf_lambda_mode mode, const int32_t* targets, int32_t n_sel, rf_product product, float* d_W,
                   void* d_W_lp, float* d_b, int32_t* d_info, double* d_cond, double* d_resid, void* d_ws,
                   size_t ws_bytes, void* stream) {
    clear_error();
    return solve_impl(desc, d_state, lambdas, n_lambda, mode, targets, n_sel, product, d_W, d_W_lp, d_b, d_info, d_cond,
                      d_resid, d_ws, ws_bytes, stream, 0);
}

rf_status rf_solve_headwise(const rf_gram_desc* desc, const void* d_state, const double* lambdas, int32_t n_lambda,
                            rf_lambda_mode mode, int32_t head_dim, const int32_t* targets, int32_t n_sel,
                            rf_product product, float* d_W, void* d_W_lp, float* d_b, int32_t* d_info, double* d_cond,
                            double* d_resid, void* d_ws, size_t ws_bytes, void* stream) {
    clear_error();
    RF_REQUIRE(desc, RF_ERR_INVALID_ARG, "rf_solve_headwise: null descriptor");
    const int64_t dy = gram_dy(desc);
    RF_REQUIRE(head_dim > 0 && head_dim % 8 == 0 && dy > 0 && dy % head_dim == 0 && desc->d % dy == 0,
               RF_ERR_INVALID_ARG,
               "rf_solve_headwise: head_dim must be a positive multiple of 8 dividing the targets' width, and d a "
               "multiple of that width (whole source layers of the same heads)");
    return solve_impl(desc, d_state, lambdas, n_lambda, mode, targets, n_sel, product, d_W, d_W_lp, d_b, d_info, d_cond,
                      d_resid, d_ws, ws_bytes, stream, head_dim);
}

}  // extern "C"
