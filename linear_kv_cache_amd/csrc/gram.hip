// One streaming pass of second moments over calibration chunks (RidgeFill project page,
// "Method" step 2: the maps are fitted in closed form from one pass over calibration text).
//
// A single launch covers every output tile of one chunk:
//   S_xx tiles (upper triangle of X^T X, by 256 x 256 tiles) and S_yx tiles (Y_l^T X).
// Both operands are calibration rows [rows][d] read column-blocks at a time (M-major), so the
// tile loop transposes 8 x 8 (bf16) or 4 x 4 (fp32) blocks in registers on their way to LDS.
// The reduction dimension is the chunk's rows; a ragged row tail reads as zero.  Tiles add
// their fp32 result into the state (read-modify-write, one owner per element).
// Column sums ride along in fp64 on the operand already in registers: the S_xx tiles of the
// first tile row sum X's columns, the S_yx tiles of the first tile column sum Y's columns, so
// each column is summed exactly once, in a fixed order.
#include "rf_internal.h"
#include "rf_mfma.h"

namespace rf {

constexpr int kMaxTargets = 64;
constexpr int kGT = 256;

struct GramArgs {
    const void* X;
    int64_t ldx;
    int64_t rows;
    int64_t ldy;
    int32_t d;
    int32_t tiles_m;   // d / kGT
    int32_t n_xx;      // S_xx upper tiles
    float* Sxx;
    float* Syx;
    double* sx;
    double* sy;
    int64_t* n;
    const void* Y[kMaxTargets];
};

struct GramLayout {
    size_t off_n, off_Sxx, off_Syx, off_sx, off_sy, total;
};

static GramLayout gram_layout(int64_t d, int64_t nt) {
    GramLayout L;
    L.off_n = 0;
    L.off_Sxx = 256;
    L.off_Syx = L.off_Sxx + round_up((size_t)(d * d) * 4, 256);
    L.off_sx = L.off_Syx + round_up((size_t)(nt * d * d) * 4, 256);
    L.off_sy = L.off_sx + round_up((size_t)d * 8, 256);
    L.total = L.off_sy + round_up((size_t)(nt * d) * 8, 256);
    return L;
}

template <typename T, int V>
__device__ inline void add_colsums(double (&cs)[V], double* dst) {
    // lanes t, t^1, t^2, t^4 hold partial sums of the same columns (different k-blocks)
#pragma unroll
    for (int v = 0; v < V; ++v) {
        double s = cs[v];
        s += __shfl_xor(s, 1);
        s += __shfl_xor(s, 2);
        s += __shfl_xor(s, 4);
        cs[v] = s;
    }
    constexpr int EPV = ElemTraits<T>::kPerVec;
    constexpr int NJ = V / EPV;
    const int t = threadIdx.x;
    if ((t & 7) == 0) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int mb = (t >> 3) + 32 * j;
#pragma unroll
            for (int i = 0; i < EPV; ++i) dst[mb * EPV + i] += cs[j * EPV + i];
        }
    }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void k_gram(GramArgs a) {
    using G = TileGemm<T, kGT, kGT, true, true>;
    __shared__ __attribute__((aligned(16))) char lds[G::LDS_BYTES];
    int bid = blockIdx.x;
    bool is_xx = bid < a.n_xx;
    int mt, nt;  // A tile = X columns [mt*256, +256); B tile = rows of S [nt*256, +256)
    if (is_xx) {
        nt = 0;
        int rem = bid;
        while (rem >= a.tiles_m - nt) {
            rem -= a.tiles_m - nt;
            ++nt;
        }
        mt = nt + rem;
    } else {
        const int j = bid - a.n_xx;
        mt = j % a.tiles_m;
        nt = j / a.tiles_m;
    }
    const int64_t srow0 = (int64_t)nt * kGT;  // first S row of this tile
    const Operand A{(const T*)a.X + (int64_t)mt * kGT, a.ldx, a.rows};
    const void* bptr;
    int64_t bld;
    if (is_xx) {
        bptr = (const T*)a.X + srow0;
        bld = a.ldx;
    } else {
        const int l = (int)(srow0 / a.d);
        bptr = (const T*)a.Y[l] + (srow0 % a.d);
        bld = a.ldy;
    }
    const Operand B{bptr, bld, a.rows};
    const int nk = (int)ceil_div(a.rows, G::BK);
    G gm;
    if (is_xx && nt == 0) {
        double cs[G::VA];
#pragma unroll
        for (int v = 0; v < G::VA; ++v) cs[v] = 0.0;
        gm.template run<true, false>(lds, A, B, nk, &cs, nullptr);
        add_colsums<T, G::VA>(cs, a.sx + (int64_t)mt * kGT);
    } else if (!is_xx && mt == 0) {
        double cs[G::VB];
#pragma unroll
        for (int v = 0; v < G::VB; ++v) cs[v] = 0.0;
        gm.template run<false, true>(lds, A, B, nk, nullptr, &cs);
        add_colsums<T, G::VB>(cs, a.sy + srow0);
    } else {
        gm.run(lds, A, B, nk);
    }
    if (bid == 0 && threadIdx.x == 0) *a.n += a.rows;

    float* S = is_xx ? a.Sxx : a.Syx;
#pragma unroll
    for (int j = 0; j < G::SN; ++j) {
        const int64_t srow = srow0 + G::col_of(j);
#pragma unroll
        for (int i = 0; i < G::SM; ++i) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t col = (int64_t)mt * kGT + G::row_of(i, 4 * q);
                f32x4* p = (f32x4*)(S + srow * a.d + col);
                f32x4 v = *p;
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] += gm.acc[i][j][4 * q + e];
                *p = v;
            }
        }
    }
}

__global__ void k_zero_bytes(uint4* p, int64_t n16) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = uint4{0u, 0u, 0u, 0u};
}

static rf_status check_desc(const rf_gram_desc* desc) {
    RF_REQUIRE(desc, RF_ERR_INVALID_ARG, "gram: null descriptor");
    RF_REQUIRE(valid_dtype(desc->dtype), RF_ERR_INVALID_ARG, "gram: bad dtype");
    RF_REQUIRE(desc->d > 0 && desc->n_targets >= 0, RF_ERR_INVALID_ARG, "gram: d must be > 0, n_targets >= 0");
    RF_REQUIRE(desc->d % kGT == 0, RF_ERR_UNSUPPORTED, "gram: d must be a multiple of 256");
    RF_REQUIRE(desc->n_targets <= kMaxTargets, RF_ERR_UNSUPPORTED, "gram: at most 64 target layers");
    return RF_OK;
}

}  // namespace rf

using namespace rf;

extern "C" {

rf_status rf_gram_state_layout(const rf_gram_desc* desc, rf_gram_layout_t* out) {
    clear_error();
    rf_status st = check_desc(desc);
    if (st != RF_OK) return st;
    RF_REQUIRE(out, RF_ERR_INVALID_ARG, "rf_gram_state_layout: null output");
    const GramLayout L = gram_layout(desc->d, desc->n_targets);
    out->off_n = (int64_t)L.off_n;
    out->off_S_xx = (int64_t)L.off_Sxx;
    out->off_S_yx = (int64_t)L.off_Syx;
    out->off_s_x = (int64_t)L.off_sx;
    out->off_s_y = (int64_t)L.off_sy;
    out->total_bytes = (int64_t)L.total;
    return RF_OK;
}

size_t rf_gram_state_bytes(const rf_gram_desc* desc) {
    rf_gram_layout_t L;
    if (rf_gram_state_layout(desc, &L) != RF_OK) return 0;
    return (size_t)L.total_bytes;
}

rf_status rf_gram_init(const rf_gram_desc* desc, void* d_state, void* stream) {
    clear_error();
    rf_status st = check_desc(desc);
    if (st != RF_OK) return st;
    RF_REQUIRE(d_state && aligned(d_state, 256), RF_ERR_INVALID_ARG, "rf_gram_init: state must be non-null, 256-B aligned");
    const GramLayout L = gram_layout(desc->d, desc->n_targets);
    const int64_t n16 = (int64_t)(L.total / 16);
    const int blocks = (int)std::min<int64_t>(ceil_div(n16, 256), 4096);
    hipLaunchKernelGGL(k_zero_bytes, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (uint4*)d_state, n16);
    return check_launch("rf_gram_init");
}

rf_status rf_gram_accumulate(const rf_gram_desc* desc, void* d_state, const void* d_X, int64_t ldx,
                             const void* const* d_Y, int64_t ldy, int64_t rows, void* stream) {
    clear_error();
    rf_status st = check_desc(desc);
    if (st != RF_OK) return st;
    RF_REQUIRE(rows >= 0, RF_ERR_INVALID_ARG, "rf_gram_accumulate: rows must be >= 0");
    RF_REQUIRE(d_state && aligned(d_state, 256), RF_ERR_INVALID_ARG, "rf_gram_accumulate: state must be non-null, 256-B aligned");
    if (rows == 0) return RF_OK;
    const size_t eb = elem_bytes(desc->dtype);
    RF_REQUIRE(d_X && aligned(d_X, 16) && ldx >= desc->d && (ldx * (int64_t)eb) % 16 == 0, RF_ERR_INVALID_ARG,
               "rf_gram_accumulate: X must be non-null, 16-B aligned, ldx >= d with 16-B row stride");
    if (desc->n_targets > 0) {
        RF_REQUIRE(d_Y && ldy >= desc->d && (ldy * (int64_t)eb) % 16 == 0, RF_ERR_INVALID_ARG,
                   "rf_gram_accumulate: Y needs n_targets pointers and ldy >= d with 16-B row stride");
        for (int l = 0; l < desc->n_targets; ++l)
            RF_REQUIRE(d_Y[l] && aligned(d_Y[l], 16), RF_ERR_INVALID_ARG, "rf_gram_accumulate: null or misaligned Y pointer");
    }
    const GramLayout L = gram_layout(desc->d, desc->n_targets);
    char* s = (char*)d_state;
    GramArgs a{};
    a.X = d_X; a.ldx = ldx; a.rows = rows; a.ldy = ldy; a.d = desc->d;
    a.tiles_m = desc->d / kGT;
    a.n_xx = a.tiles_m * (a.tiles_m + 1) / 2;
    a.Sxx = (float*)(s + L.off_Sxx); a.Syx = (float*)(s + L.off_Syx);
    a.sx = (double*)(s + L.off_sx); a.sy = (double*)(s + L.off_sy); a.n = (int64_t*)(s + L.off_n);
    for (int l = 0; l < desc->n_targets; ++l) a.Y[l] = d_Y[l];
    const int n_yx = a.tiles_m * (int)((int64_t)desc->n_targets * desc->d / kGT);
    const dim3 grid(a.n_xx + n_yx);
    if (desc->dtype == RF_BF16)
        hipLaunchKernelGGL(k_gram<bf16_t>, grid, dim3(kThreads), 0, (hipStream_t)stream, a);
    else
        hipLaunchKernelGGL(k_gram<float>, grid, dim3(kThreads), 0, (hipStream_t)stream, a);
    return check_launch("rf_gram_accumulate");
}

}  // extern "C"
