// One streaming pass of second moments over calibration chunks (RidgeFill project page,
// "Method" step 2: the maps are fitted in closed form from one pass over calibration text).
//
// bf16 chunks take one launch, k_gram_pipe:
//   - S_yx tiles (Y_l^T X) and the S_xx upper triangle (X^T X, 256 x 256 tiles) on the
//     software-pipelined bf16 MFMA core, reading X and Y_l as they lie ([rows][d]: the
//     reduction runs over rows, the core's M-major operand form), in an XCD-aware order; each
//     tile adds its fp32 result into the state (one owner per element);
//   - then, in the launch's last work-groups, exact fp64 column sums of X and every Y_l (bf16
//     values have 8-bit significands; each column is summed in one fixed order).  They run on
//     the CUs the last partial round of tiles leaves idle.
// fp32 chunks (small widths) run one launch of the plain tile loop, which transposes 4 x 4
// blocks on their way to LDS and sums the columns on the operand already in registers, and a
// small pass for the targets' column sums of squares.
// The column sums of squares of every Y_l (fp64) let the fit's R^2 be read off the state
// (rf_fit_r2) without another pass over the data.
#include "rf_internal.h"
#include "rf_mfma.h"
#include "rf_pipe.h"

namespace rf {

constexpr int kMaxTargets = 64;
constexpr int kGT = 256;

struct GramArgs {
    const void* X;
    int64_t ldx;
    int64_t rows;
    int64_t ldy;
    int32_t d;
    int32_t dy;        // width of each target's rows
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
    size_t off_n, off_Sxx, off_Syx, off_sx, off_sy, off_syy, total;
};

static GramLayout gram_layout(int64_t d, int64_t nt, int64_t dy) {
    GramLayout L;
    L.off_n = 0;
    L.off_Sxx = 256;
    L.off_Syx = L.off_Sxx + round_up((size_t)(d * d) * 4, 256);
    L.off_sx = L.off_Syx + round_up((size_t)(nt * dy * d) * 4, 256);
    L.off_sy = L.off_sx + round_up((size_t)d * 8, 256);
    L.off_syy = L.off_sy + round_up((size_t)(nt * dy) * 8, 256);
    L.total = L.off_syy + round_up((size_t)(nt * dy) * 8, 256);
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
        const int l = (int)(srow0 / a.dy);
        bptr = (const T*)a.Y[l] + (srow0 % a.dy);
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

// ---- bf16: column sums ------------------------------------------------------------------------
struct ColsumArgs {
    const void* src[kMaxTargets + 1];   // [rows][ld] per matrix: X, then Y_0 .. Y_{L-1}
    int64_t ld[kMaxTargets + 1];
    double* csum[kMaxTargets + 1];      // column sums to add into: s_x, then s_y + l*dy
    double* csq[kMaxTargets + 1];       // column sums of squares (null for X): s_yy + l*dy
    int64_t rows;
    int32_t blocks_x;                   // d / 64 work-groups for X
    int32_t blocks_y;                   // dy / 64 work-groups for each Y_l
};

// One work-group per 64 columns of one matrix (X first, then each Y_l): thread t sums columns 8 (t & 7) .. + 8 over rows
// r = t >> 3 (mod 32) in ascending order (eight rows in flight), then the 32 row groups are added
// in a fixed order: the result does not depend on scheduling.
// red: LDS of at least 2 * 32 * 65 doubles.
__device__ inline void colsum_block(const ColsumArgs& a, int b, double (*red)[32][64 + 1]) {
    const int by = b - a.blocks_x;
    const int g = by < 0 ? 0 : 1 + by / a.blocks_y;
    const int c0 = (by < 0 ? b : by % a.blocks_y) * 64;
    const int t = threadIdx.x, ch = t & 7, rg = t >> 3;
    const int64_t ld = a.ld[g];
    const bf16_t* src = (const bf16_t*)a.src[g] + c0 + ch * 8;
    const bool sq = g > 0;   // targets also carry sums of squares (uniform per work-group)
    double s[8], s2[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] = s2[e] = 0.0;
    auto add = [&](const u32x4& v) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const double lo = (double)__uint_as_float(v[w] << 16), hi = (double)__uint_as_float(v[w] & 0xffff0000u);
            s[2 * w] += lo;
            s[2 * w + 1] += hi;
            if (sq) {
                s2[2 * w] += lo * lo;
                s2[2 * w + 1] += hi * hi;
            }
        }
    };
    int64_t r = rg;
    for (; r + 7 * 32 < a.rows; r += 8 * 32) {
        u32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = *(const u32x4*)(src + (r + 32 * u) * ld);
#pragma unroll
        for (int u = 0; u < 8; ++u) add(v[u]);
    }
    for (; r < a.rows; r += 32) add(*(const u32x4*)(src + r * ld));
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        red[0][rg][ch * 8 + e] = s[e];
        red[1][rg][ch * 8 + e] = s2[e];
    }
    __syncthreads();
    if (t < 64) {
        double x = 0.0;
        for (int q = 0; q < 32; ++q) x += red[0][q][t];
        a.csum[g][c0 + t] += x;
    } else if (t < 128 && sq) {
        double x = 0.0;
        for (int q = 0; q < 32; ++q) x += red[1][q][t - 64];
        a.csq[g][c0 + t - 64] += x;
    }
}

// fp32 chunks: column sums of squares of every Y_l, one thread per column, rows in order.
__global__ void k_sqsum_f32(ColsumArgs a) {
    const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // over n_targets * dy
    const int64_t dy = (int64_t)a.blocks_y * 64;
    const int l = (int)(c / dy);
    if (l >= a.blocks_x) return;   // blocks_x holds the number of targets here
    const int64_t o = c - l * dy;
    const float* src = (const float*)a.src[l + 1] + o;
    double x = 0.0;
    for (int64_t r = 0; r < a.rows; ++r) {
        const double v = (double)src[r * a.ld[l + 1]];
        x += v * v;
    }
    a.csq[l + 1][o] += x;
}

// ---- bf16: products on the pipelined core ----------------------------------------------------
struct PipeGramArgs {
    const bf16_t* X;        // [rows][ldx]
    int64_t ldx;
    const bf16_t* Y[kMaxTargets];   // [rows][ldy] each
    int64_t ldy;
    int64_t rows;           // rows of this piece (the reduction extent; also added to n)
    int32_t d;
    int32_t dy;             // width of each Y_l
    int32_t tiles_m;        // d / 256
    int32_t n_xx;           // S_xx upper tiles
    int32_t n_yx;           // S_yx tiles
    float* Sxx;
    float* Syx;
    int64_t* n;
};

// Logical tiles [0, n_yx) are S_yx tiles, walked in groups of 4 X tiles x 8 Y tiles per XCD
// step; [n_yx, n_yx + n_xx) are the S_xx upper triangle.  MFMA operand A = X^T rows (X column
// tile mt), B = rows of the S tile (Y_l^T or X^T), so each lane holds 4 consecutive columns of
// one S row: one 16-byte read-modify-write.
using GramCore = PipeGemmW<4, 2, true>;

// Work-groups past the product tiles compute the column sums (colsum_block): dispatched last,
// they run on the CUs the last partial round of tiles leaves idle.
__global__ __launch_bounds__(GramCore::kThr) void k_gram_pipe(PipeGramArgs a, ColsumArgs ca) {
    using G = GramCore;
    __shared__ __attribute__((aligned(16))) char lds[G::LDS_BYTES];
    const int n_tiles = a.n_yx + a.n_xx;
    if ((int)blockIdx.x >= n_tiles) {
        colsum_block(ca, (int)blockIdx.x - n_tiles, (double (*)[32][64 + 1])lds);
        return;
    }
    const int v = xcd_order((int)blockIdx.x, n_tiles);
    int mt, nt;
    const bool is_xx = v >= a.n_yx;
    if (is_xx) {
        nt = 0;
        int rem = v - a.n_yx;
        while (rem >= a.tiles_m - nt) {
            rem -= a.tiles_m - nt;
            ++nt;
        }
        mt = nt + rem;
    } else {
        grouped_tile(v, a.tiles_m, a.n_yx / a.tiles_m, 4, mt, nt);
    }
    const int64_t srow0 = (int64_t)nt * kGT;
    const bf16_t* Bp;
    int64_t ldb;
    if (is_xx) {
        Bp = a.X + srow0;
        ldb = a.ldx;
    } else {
        Bp = a.Y[srow0 / a.dy] + srow0 % a.dy;
        ldb = a.ldy;
    }
    int nk = (int)((a.rows + G::BK - 1) / G::BK);
    nk += nk & 1;   // the core takes k-steps in pairs; rows past the end read as zero
    G gm;
    gm.run(lds, PipeOperand{a.X + (int64_t)mt * kGT, a.ldx, a.rows}, PipeOperand{Bp, ldb, a.rows}, nk);
    if (v == 0 && threadIdx.x == 0) *a.n += a.rows;
    // Read-modify-write of the S tile, one 32-row block at a time: all 16 reads of a block are
    // issued before its writes (a store followed by a load the compiler cannot prove disjoint
    // would otherwise cost one full memory round trip per 16 bytes).
    float* S = is_xx ? a.Sxx : a.Syx;
#pragma unroll
    for (int j = 0; j < G::SN; ++j) {
        float* srow = S + (srow0 + G::col_of(j)) * a.d + (int64_t)mt * kGT;
        f32x4 x[G::SM][4];
#pragma unroll
        for (int i = 0; i < G::SM; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) x[i][q] = *(const f32x4*)(srow + G::row_of(i, 4 * q));
#pragma unroll
        for (int i = 0; i < G::SM; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
#pragma unroll
                for (int e = 0; e < 4; ++e) x[i][q][e] += gm.acc[i][j][4 * q + e];
                *(f32x4*)(srow + G::row_of(i, 4 * q)) = x[i][q];
            }
    }
}

__global__ void k_zero_bytes(uint4* p, int64_t n16) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = uint4{0u, 0u, 0u, 0u};
}

// ---- sub-states of column blocks ----------------------------------------------------------
constexpr int kMaxSelBlocks = 64;
struct SelectArgs {
    int32_t blk[kMaxSelBlocks];   // selected source blocks, ascending
    int32_t bw;                   // block width (columns)
};

// dst[r][c] = src[R(r)][C(c)] with C mapping destination column block c / bw to source block
// blk[c / bw] (and R the same for rows when map_rows), 4 columns per thread.
__global__ void k_select_cols(const float* __restrict__ src, int64_t lds, float* __restrict__ dst, int64_t ldd,
                              int64_t rows, int64_t cols, int map_rows, SelectArgs s) {
    const int64_t c4 = cols / 4;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < rows * c4;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = i / c4, c = (i - r * c4) * 4;
        const int64_t sr = map_rows ? (int64_t)s.blk[r / s.bw] * s.bw + r % s.bw : r;
        const int64_t sc = (int64_t)s.blk[c / s.bw] * s.bw + c % s.bw;
        *(f32x4*)(dst + r * ldd + c) = *(const f32x4*)(src + sr * lds + sc);
    }
}

// n, the selected entries of s_x, and s_y, s_yy as they are.
__global__ void k_select_vecs(const int64_t* n, const double* sx, const double* sy, const double* syy, int64_t dx,
                              int64_t ny, int64_t* n_out, double* sx_out, double* sy_out, double* syy_out,
                              SelectArgs s) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < dx + ny;
         i += (int64_t)gridDim.x * blockDim.x) {
        if (i < dx) {
            sx_out[i] = sx[(int64_t)s.blk[i / s.bw] * s.bw + i % s.bw];
        } else {
            sy_out[i - dx] = sy[i - dx];
            syy_out[i - dx] = syy[i - dx];
        }
        if (i == 0) *n_out = *n;
    }
}

static rf_status check_desc(const rf_gram_desc* desc) {
    RF_REQUIRE(desc, RF_ERR_INVALID_ARG, "gram: null descriptor");
    RF_REQUIRE(valid_dtype(desc->dtype), RF_ERR_INVALID_ARG, "gram: bad dtype");
    RF_REQUIRE(desc->d > 0 && desc->n_targets >= 0, RF_ERR_INVALID_ARG, "gram: d must be > 0, n_targets >= 0");
    RF_REQUIRE(desc->d % kGT == 0, RF_ERR_UNSUPPORTED, "gram: d must be a multiple of 256");
    RF_REQUIRE(desc->n_targets <= kMaxTargets, RF_ERR_UNSUPPORTED, "gram: at most 64 target layers");
    RF_REQUIRE(desc->d_out >= 0, RF_ERR_INVALID_ARG, "gram: d_out must be >= 0");
    RF_REQUIRE(desc->d_out % kGT == 0 && desc->d_out <= (1 << 16), RF_ERR_UNSUPPORTED,
               "gram: d_out must be 0 or a multiple of 256, at most 65536");
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
    const GramLayout L = gram_layout(desc->d, desc->n_targets, gram_dy(desc));
    out->off_n = (int64_t)L.off_n;
    out->off_S_xx = (int64_t)L.off_Sxx;
    out->off_S_yx = (int64_t)L.off_Syx;
    out->off_s_x = (int64_t)L.off_sx;
    out->off_s_y = (int64_t)L.off_sy;
    out->off_s_yy = (int64_t)L.off_syy;
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
    const GramLayout L = gram_layout(desc->d, desc->n_targets, gram_dy(desc));
    const int64_t n16 = (int64_t)(L.total / 16);
    const int blocks = (int)std::min<int64_t>(ceil_div(n16, 256), 4096);
    hipLaunchKernelGGL(k_zero_bytes, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (uint4*)d_state, n16);
    return check_launch("rf_gram_init");
}

rf_status rf_gram_select(const rf_gram_desc* desc, const void* d_state, int32_t block_width, const int32_t* blocks,
                         int32_t n_sel, const rf_gram_desc* desc_out, void* d_state_out, void* stream) {
    clear_error();
    rf_status st = check_desc(desc);
    if (st != RF_OK) return st;
    st = check_desc(desc_out);
    if (st != RF_OK) return st;
    RF_REQUIRE(block_width > 0 && block_width % kGT == 0 && desc->d % block_width == 0, RF_ERR_UNSUPPORTED,
               "rf_gram_select: block_width must be a multiple of 256 that divides d");
    RF_REQUIRE(n_sel >= 1 && n_sel <= kMaxSelBlocks && blocks, RF_ERR_INVALID_ARG,
               "rf_gram_select: 1..64 selected blocks");
    const int32_t n_blocks = desc->d / block_width;
    for (int i = 0; i < n_sel; ++i)
        RF_REQUIRE(blocks[i] >= 0 && blocks[i] < n_blocks && (i == 0 || blocks[i] > blocks[i - 1]), RF_ERR_INVALID_ARG,
                   "rf_gram_select: block indices must ascend strictly within [0, d / block_width)");
    RF_REQUIRE(desc_out->d == (int64_t)n_sel * block_width && desc_out->n_targets == desc->n_targets &&
                   gram_dy(desc_out) == gram_dy(desc) && desc_out->dtype == desc->dtype,
               RF_ERR_INVALID_ARG, "rf_gram_select: desc_out must have d = n_sel * block_width and the same targets");
    RF_REQUIRE(d_state && d_state_out && aligned(d_state, 256) && aligned(d_state_out, 256) && d_state != d_state_out,
               RF_ERR_INVALID_ARG, "rf_gram_select: states must be distinct, non-null and 256-B aligned");
    const GramLayout Ls = gram_layout(desc->d, desc->n_targets, gram_dy(desc));
    const GramLayout Ld = gram_layout(desc_out->d, desc_out->n_targets, gram_dy(desc_out));
    const char* s = (const char*)d_state;
    char* o = (char*)d_state_out;
    SelectArgs sa{};
    for (int i = 0; i < n_sel; ++i) sa.blk[i] = blocks[i];
    sa.bw = block_width;
    hipStream_t strm = (hipStream_t)stream;
    const int64_t dd = desc_out->d, ny = (int64_t)desc->n_targets * gram_dy(desc);
    auto grid = [](int64_t n) { return dim3((unsigned)std::min<int64_t>(std::max<int64_t>(ceil_div(n, 256), 1), 8192)); };
    // ascending blocks keep every selected upper-triangle block in the source's upper triangle
    hipLaunchKernelGGL(k_select_cols, grid(dd * dd / 4), dim3(256), 0, strm, (const float*)(s + Ls.off_Sxx),
                       (int64_t)desc->d, (float*)(o + Ld.off_Sxx), dd, dd, dd, 1, sa);
    st = check_launch("rf_gram_select: S_xx");
    if (st != RF_OK) return st;
    if (ny > 0) {
        hipLaunchKernelGGL(k_select_cols, grid(ny * dd / 4), dim3(256), 0, strm, (const float*)(s + Ls.off_Syx),
                           (int64_t)desc->d, (float*)(o + Ld.off_Syx), dd, ny, dd, 0, sa);
        st = check_launch("rf_gram_select: S_yx");
        if (st != RF_OK) return st;
    }
    hipLaunchKernelGGL(k_select_vecs, grid(dd + ny), dim3(256), 0, strm, (const int64_t*)(s + Ls.off_n),
                       (const double*)(s + Ls.off_sx), (const double*)(s + Ls.off_sy), (const double*)(s + Ls.off_syy),
                       dd, ny, (int64_t*)(o + Ld.off_n), (double*)(o + Ld.off_sx), (double*)(o + Ld.off_sy),
                       (double*)(o + Ld.off_syy), sa);
    return check_launch("rf_gram_select: sums");
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
    const int64_t dy = gram_dy(desc);
    if (desc->n_targets > 0) {
        RF_REQUIRE(d_Y && ldy >= dy && (ldy * (int64_t)eb) % 16 == 0, RF_ERR_INVALID_ARG,
                   "rf_gram_accumulate: Y needs n_targets pointers and ldy >= d_out with 16-B row stride");
        for (int l = 0; l < desc->n_targets; ++l)
            RF_REQUIRE(d_Y[l] && aligned(d_Y[l], 16), RF_ERR_INVALID_ARG, "rf_gram_accumulate: null or misaligned Y pointer");
    }
    const GramLayout L = gram_layout(desc->d, desc->n_targets, dy);
    char* s = (char*)d_state;
    hipStream_t strm = (hipStream_t)stream;
    float* Sxx = (float*)(s + L.off_Sxx);
    float* Syx = (float*)(s + L.off_Syx);
    double* sx = (double*)(s + L.off_sx);
    double* sy = (double*)(s + L.off_sy);
    double* syy = (double*)(s + L.off_syy);
    int64_t* np = (int64_t*)(s + L.off_n);
    const int tiles_m = desc->d / kGT;
    const int n_xx = tiles_m * (tiles_m + 1) / 2;
    const int n_yx = tiles_m * (int)((int64_t)desc->n_targets * dy / kGT);

    if (desc->dtype == RF_F32) {
        GramArgs a{};
        a.X = d_X; a.ldx = ldx; a.rows = rows; a.ldy = ldy; a.d = desc->d; a.dy = (int32_t)dy;
        a.tiles_m = tiles_m; a.n_xx = n_xx;
        a.Sxx = Sxx; a.Syx = Syx; a.sx = sx; a.sy = sy; a.n = np;
        for (int l = 0; l < desc->n_targets; ++l) a.Y[l] = d_Y[l];
        hipLaunchKernelGGL(k_gram<float>, dim3(n_xx + n_yx), dim3(kThreads), 0, strm, a);
        st = check_launch("rf_gram_accumulate");
        if (st != RF_OK || desc->n_targets == 0) return st;
        ColsumArgs qa{};
        for (int l = 0; l < desc->n_targets; ++l) {
            qa.src[l + 1] = d_Y[l]; qa.ld[l + 1] = ldy; qa.csq[l + 1] = syy + (int64_t)l * dy;
        }
        qa.rows = rows; qa.blocks_x = desc->n_targets; qa.blocks_y = (int32_t)(dy / 64);
        hipLaunchKernelGGL(k_sqsum_f32, dim3((unsigned)ceil_div(desc->n_targets * dy, 256)), dim3(256), 0, strm, qa);
        return check_launch("rf_gram_accumulate: sums of squares");
    }

    // bf16: pieces small enough for 32-bit byte offsets into X and Y (the products address a
    // whole piece from the start of its rows)
    const int64_t ld_max = std::max<int64_t>(ldx, desc->n_targets > 0 ? ldy : 0);
    const int64_t lim = (((int64_t)1 << 31) - 1);
    const int64_t cap = (lim / (ld_max * 2) - 64) / 64 * 64;
    RF_REQUIRE(cap >= 64, RF_ERR_UNSUPPORTED, "rf_gram_accumulate: row stride too large for 32-bit offsets");
    for (int64_t r0 = 0; r0 < rows; r0 += cap) {
        const int64_t pr = std::min(cap, rows - r0);
        ColsumArgs ca{};
        ca.src[0] = (const bf16_t*)d_X + r0 * ldx; ca.ld[0] = ldx; ca.csum[0] = sx;
        for (int l = 0; l < desc->n_targets; ++l) {
            ca.src[l + 1] = (const bf16_t*)d_Y[l] + r0 * ldy; ca.ld[l + 1] = ldy; ca.csum[l + 1] = sy + (int64_t)l * dy;
            ca.csq[l + 1] = syy + (int64_t)l * dy;
        }
        ca.rows = pr; ca.blocks_x = desc->d / 64; ca.blocks_y = (int32_t)(dy / 64);
        const int n_colsum = ca.blocks_x + desc->n_targets * ca.blocks_y;
        PipeGramArgs pa{};
        pa.X = (const bf16_t*)d_X + r0 * ldx; pa.ldx = ldx;
        for (int l = 0; l < desc->n_targets; ++l) pa.Y[l] = (const bf16_t*)d_Y[l] + r0 * ldy;
        pa.ldy = ldy; pa.rows = pr; pa.d = desc->d; pa.dy = (int32_t)dy; pa.tiles_m = tiles_m;
        pa.n_xx = n_xx; pa.n_yx = n_yx; pa.Sxx = Sxx; pa.Syx = Syx; pa.n = np;
        hipLaunchKernelGGL(k_gram_pipe, dim3((unsigned)(n_xx + n_yx + n_colsum)), dim3(GramCore::kThr), 0, strm, pa, ca);
        st = check_launch("rf_gram_accumulate: products");
        if (st != RF_OK) return st;
    }
    return RF_OK;
}

}  // extern "C"
