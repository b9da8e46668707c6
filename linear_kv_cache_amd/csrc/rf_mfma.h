// MFMA GEMM core for gfx950 shared by the fill and Gram kernels.
//
// One workgroup computes a BM x BN tile of  acc[m][n] = sum_k A[m][k] * B[n][k]  with 256
// threads (4 waves in a 2 x 2 grid).  Each wave owns a (BM/2) x (BN/2) sub-tile made of
// 32 x 32 MFMA blocks; fp32 accumulators live in the unified register file.
//
// Operands are read from HBM one k-tile (128 bytes of K per row) at a time with 16-byte
// vector loads and staged in LDS, double-buffered: the next k-tile is in flight in
// registers while MFMAs consume the current one, so one barrier per k-tile suffices.
//   * K-major operand  (row m contiguous in k): loaded as is.
//   * M-major operand  (global [k][m], m contiguous): each thread loads a 16-byte x
//     (16 / elem) block and transposes it in registers before the LDS write, so LDS always
//     holds rows of K and the MFMA fragment reads are identical for both kinds.
// LDS rows are 128 bytes plus 16 bytes of padding (stride 144 B): 16 consecutive rows then
// start on 16 distinct 4-bank groups, so the 16-byte fragment reads are conflict-free.
//
// MFMA lane layout (v_mfma_f32_32x32x16_bf16 and v_mfma_f32_32x32x2_f32): lane l supplies
// row (l % 32) of A and of B and half (l / 32) of the 32-byte k-slice; accumulator register
// i of lane l holds C[m = 8*(i/4) + 4*(l/32) + i%4][n = l % 32].  A k-permutation shared by
// both operands leaves the sum unchanged, so the exact intra-instruction k order is not
// relied upon.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rf {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kRowBytes = 128;   // bytes of K per LDS row per k-tile
constexpr int kLdsStride = 144;  // padded LDS row stride in bytes
constexpr int kThreads = 256;

// bf16 is carried as raw 16-bit words in memory.
typedef uint16_t bf16_t;

template <typename T> struct ElemTraits;
template <> struct ElemTraits<bf16_t> {
    static constexpr int kPerVec = 8;  // elements per 16-byte vector
    __device__ static inline float to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }
};
template <> struct ElemTraits<float> {
    static constexpr int kPerVec = 4;
    __device__ static inline float to_f32(uint32_t bits) { return __uint_as_float(bits); }
};

// f as an fp32 value the compiler must materialise.  A double narrowed to fp32 and then to bf16
// is rounded twice, as the fp32 copy of the same value is; without the barrier the compiler
// may fuse the two narrowings into one rounding from the double (which can differ in the last
// bf16 bit from rounding the stored fp32 value).
__device__ inline float opaque_f32(float f) {
    __asm__("" : "+v"(f));
    return f;
}

__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
    __bf16 a = (__bf16)lo;  // round to nearest even (v_cvt_pk_bf16_f32)
    __bf16 b = (__bf16)hi;
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// One 32-byte k-slice of MFMA work on 16-byte fragments.
template <typename T> struct MfmaStep;
template <> struct MfmaStep<bf16_t> {
    __device__ static inline void run(f32x16& c, const u32x4& a, const u32x4& b) {
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
};
template <> struct MfmaStep<float> {
    __device__ static inline void run(f32x16& c, const u32x4& a, const u32x4& b) {
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
    }
};

// Transpose of a (16/elem) x (16/elem) block held as one 16-byte vector per k-row into one
// 16-byte vector per m-column.
template <typename T> struct Transpose;
template <> struct Transpose<bf16_t> {
    __device__ static inline void run(const u32x4 (&in)[8], u32x4 (&out)[8]) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int w = i >> 1;
            const bool hi = i & 1;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                uint32_t a = in[2 * p][w];
                uint32_t b = in[2 * p + 1][w];
                out[i][p] = hi ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
            }
        }
    }
};
template <> struct Transpose<float> {
    __device__ static inline void run(const u32x4 (&in)[4], u32x4 (&out)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) out[i][r] = in[r][i];
    }
};

// Operand of the tile loop.
//   KMAJOR: ptr -> element (row 0 of the tile, k = 0); row r at ptr + r*ld; rows at or past
//           ``valid`` are clamped to valid-1 (in-bounds reads whose results are discarded).
//   MMAJOR: ptr -> element (k = 0, column 0 of the tile); k-row k at ptr + k*ld; k-rows at or
//           past ``valid`` read as zero (ragged K tails contribute nothing).
struct Operand {
    const void* ptr;
    int64_t ld;
    int64_t valid;
};

template <typename T, int BM, int BN, bool A_MMAJOR, bool B_MMAJOR>
struct TileGemm {
    static constexpr int kThr = kThreads;
    static constexpr int WGN = 2;  // waves per row of the 2 x 2 wave grid
    static constexpr int EPV = ElemTraits<T>::kPerVec;
    static constexpr int BK = kRowBytes / (int)sizeof(T);
    static constexpr int WTM = BM / 2, WTN = BN / 2;
    static constexpr int SM = WTM / 32, SN = WTN / 32;
    static constexpr int STAGE_BYTES = (BM + BN) * kLdsStride;
    static constexpr int LDS_BYTES = 2 * STAGE_BYTES;
    // per-thread 16-byte vectors per operand per k-tile
    static constexpr int VA = BM * 8 / kThreads;
    static constexpr int VB = BN * 8 / kThreads;
    static_assert(BM % 64 == 0 && BN % 64 == 0, "tile must split into 32x32 blocks per wave");
    static_assert(!A_MMAJOR || (BM / EPV) % 32 == 0, "M-major tile width");
    static_assert(!B_MMAJOR || (BN / EPV) % 32 == 0, "M-major tile width");

    f32x16 acc[SM][SN];

    __device__ inline void zero() {
#pragma unroll
        for (int i = 0; i < SM; ++i)
#pragma unroll
            for (int j = 0; j < SN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    }

    // ---- global -> registers ------------------------------------------------------------
    template <int R, int V, bool MMAJOR>
    __device__ static inline void load(const Operand& op, int kt, u32x4 (&reg)[V]) {
        const int t = threadIdx.x;
        if constexpr (!MMAJOR) {
            const char* base = (const char*)op.ptr + (int64_t)kt * kRowBytes;
#pragma unroll
            for (int j = 0; j < V; ++j) {
                int64_t row = j * (kThreads / 8) + (t >> 3);
                row = row < op.valid ? row : op.valid - 1;
                reg[j] = *(const u32x4*)(base + row * op.ld * (int64_t)sizeof(T) + (t & 7) * 16);
            }
        } else {
            // V == EPV * (R / EPV / 32): blocks of EPV k-rows x EPV columns
            constexpr int NJ = R / EPV / 32;
            const int kb = t & 7;
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int mb = (t >> 3) + 32 * j;
#pragma unroll
                for (int r = 0; r < EPV; ++r) {
                    const int64_t k = (int64_t)kt * BK + kb * EPV + r;
                    if (k < op.valid)
                        reg[j * EPV + r] = *(const u32x4*)((const char*)op.ptr +
                                                          (k * op.ld + (int64_t)mb * EPV) * (int64_t)sizeof(T));
                    else
                        reg[j * EPV + r] = u32x4{0u, 0u, 0u, 0u};
                }
            }
        }
    }

    // ---- registers -> LDS -----------------------------------------------------------------
    template <int R, int V, bool MMAJOR>
    __device__ static inline void store(char* lds, const u32x4 (&reg)[V]) {
        const int t = threadIdx.x;
        if constexpr (!MMAJOR) {
#pragma unroll
            for (int j = 0; j < V; ++j) {
                const int row = j * (kThreads / 8) + (t >> 3);
                *(u32x4*)(lds + row * kLdsStride + (t & 7) * 16) = reg[j];
            }
        } else {
            constexpr int NJ = R / EPV / 32;
            const int kb = t & 7;
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int mb = (t >> 3) + 32 * j;
                u32x4 in[EPV], out[EPV];
#pragma unroll
                for (int r = 0; r < EPV; ++r) in[r] = reg[j * EPV + r];
                Transpose<T>::run(in, out);
#pragma unroll
                for (int i = 0; i < EPV; ++i)
                    *(u32x4*)(lds + (mb * EPV + i) * kLdsStride + kb * 16) = out[i];
            }
        }
    }

    // Column sums over the k-tile of an M-major operand held in registers (EPV columns per
    // 16-byte vector, NJ groups); added into fp64 accumulators.
    template <int R, int V>
    __device__ static inline void colsum(const u32x4 (&reg)[V], double (&cs)[V]) {
        constexpr int NJ = R / EPV / 32;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
#pragma unroll
            for (int i = 0; i < EPV; ++i) {
                double s = cs[j * EPV + i];
#pragma unroll
                for (int r = 0; r < EPV; ++r) {
                    uint32_t w = reg[j * EPV + r][i * (int)sizeof(T) / 4];
                    if constexpr (sizeof(T) == 2) w = (i & 1) ? (w >> 16) : (w & 0xffffu);
                    s += (double)ElemTraits<T>::to_f32(w);  // exact: fp64 holds every partial sum
                }
                cs[j * EPV + i] = s;
            }
        }
    }

    // ---- MFMAs on one LDS stage -----------------------------------------------------------
    __device__ inline void compute(const char* stage) {
        const int lane = threadIdx.x & 63;
        const int wave = threadIdx.x >> 6;
        const int wm = wave >> 1, wn = wave & 1;
        const char* As = stage + (wm * WTM + (lane & 31)) * kLdsStride + (lane >> 5) * 16;
        const char* Bs = stage + (BM + wn * WTN + (lane & 31)) * kLdsStride + (lane >> 5) * 16;
#pragma unroll
        for (int kk = 0; kk < kRowBytes / 32; ++kk) {
            u32x4 a[SM], b[SN];
#pragma unroll
            for (int i = 0; i < SM; ++i) a[i] = *(const u32x4*)(As + i * 32 * kLdsStride + kk * 32);
#pragma unroll
            for (int j = 0; j < SN; ++j) b[j] = *(const u32x4*)(Bs + j * 32 * kLdsStride + kk * 32);
#pragma unroll
            for (int i = 0; i < SM; ++i)
#pragma unroll
                for (int j = 0; j < SN; ++j) MfmaStep<T>::run(acc[i][j], a[i], b[j]);
        }
    }

    // Full K loop.  ``csA``/``csB`` (may be null) receive fp64 column sums of an M-major
    // operand; the sums are partial per thread and must be reduced by the caller.
    template <bool CS_A = false, bool CS_B = false>
    __device__ inline void run(char* lds, const Operand& A, const Operand& B, int nk,
                               double (*csA)[VA] = nullptr, double (*csB)[VB] = nullptr) {
        u32x4 ra[VA], rb[VB];
        zero();
        if (nk <= 0) return;
        load<BM, VA, A_MMAJOR>(A, 0, ra);
        load<BN, VB, B_MMAJOR>(B, 0, rb);
        if constexpr (CS_A) colsum<BM, VA>(ra, *csA);
        if constexpr (CS_B) colsum<BN, VB>(rb, *csB);
        store<BM, VA, A_MMAJOR>(lds, ra);
        store<BN, VB, B_MMAJOR>(lds + BM * kLdsStride, rb);
        __syncthreads();
        for (int kt = 0; kt < nk; ++kt) {
            char* cur = lds + (kt & 1) * STAGE_BYTES;
            char* nxt = lds + ((kt + 1) & 1) * STAGE_BYTES;
            const bool more = kt + 1 < nk;
            if (more) {
                load<BM, VA, A_MMAJOR>(A, kt + 1, ra);
                load<BN, VB, B_MMAJOR>(B, kt + 1, rb);
            }
            compute(cur);
            if (more) {
                if constexpr (CS_A) colsum<BM, VA>(ra, *csA);
                if constexpr (CS_B) colsum<BN, VB>(rb, *csB);
                store<BM, VA, A_MMAJOR>(nxt, ra);
                store<BN, VB, B_MMAJOR>(nxt + BM * kLdsStride, rb);
            }
            __syncthreads();
        }
    }

    // Coordinates of accumulator register r of block (i, j) for this lane, relative to the
    // tile origin.
    __device__ static inline int row_of(int i, int r) {
        const int lane = threadIdx.x & 63, wm = (threadIdx.x >> 6) >> 1;
        return wm * WTM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
    }
    __device__ static inline int col_of(int j) {
        const int lane = threadIdx.x & 63, wn = (threadIdx.x >> 6) & 1;
        return wn * WTN + j * 32 + (lane & 31);
    }
};

}  // namespace rf
