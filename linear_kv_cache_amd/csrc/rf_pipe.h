// Software-pipelined bf16 MFMA GEMM core for gfx950, used by the fill kernels.
//
// One workgroup computes a 256 x 256 tile of  acc[m][n] = sum_k A[m][k] * B[n][k]  with both
// operands K-contiguous ("K-major"), with either 4 waves (one per SIMD, 2 x 2 grid, each wave
// 128 x 128 = 4 x 4 blocks of v_mfma_f32_32x32x16_bf16 filling the 256 accumulation registers)
// or 8 waves (two per SIMD, 2 x 4 grid, each wave 128 x 64 in 128 registers): the second wave
// of a SIMD issues MFMAs while the first waits on memory.
//
// Data movement per k-step of 64 elements (128 bytes of every operand row):
//   HBM/L2 -> VGPR : buffer loads of 16 bytes per lane into one of two register sets, issued
//                    two k-steps before their LDS write (three before their use).  Rows of a
//                    ragged tail fall outside the buffer's byte range and read as zero.
//   VGPR -> LDS    : two LDS stages of 64 KiB.  A row of 128 bytes is 8 chunks of 16 bytes;
//                    chunk c of row r is stored in slot c ^ ((r >> 1) & 7).  gfx950's LDS has
//                    64 banks of 4 bytes, so a 16-byte access serves 16 lanes per cycle; the
//                    16 rows read by 16 consecutive lanes then cover all 64 banks once, and the
//                    two rows written by 16 consecutive lanes do too: no bank conflicts and no
//                    padding.
//   LDS -> VGPR    : fragments are double-buffered in registers: the reads for slice kk+1 are
//                    in flight while the 16 MFMAs of slice kk run.
// One barrier per k-step, placed half-way through the last slice: by then every wave has
// written the next stage and finished reading the current one, and the fragment reads of the
// next stage overlap the remaining MFMAs.
//
// MFMA lane layout (v_mfma_f32_32x32x16_bf16): lane l supplies row (l % 32) of A and of B and
// the 16-byte half (l / 32) of a 32-byte k-slice; accumulator register i of lane l holds
// C[m = 8*(i/4) + 4*(l/32) + i%4][n = l % 32].  The k-permutation inside a slice is the same for
// both operands, so the sum is unchanged by it.
//
// M-major operands (MMAJOR): both operands are instead stored with m contiguous and k as the row
// index (a [k][m] matrix, e.g. calibration rows x features), and the product contracts over k.
// A k-step stages 64 rows x 256 columns (512 bytes) of each operand as they lie in memory; the
// 16-byte chunk c of staged row k sits in slot c ^ 4 (k & 3).  Fragments come from gfx950's
// transposing LDS read (ds_read_b64_tr_b16): in each group of 16 lanes, source lane j points at
// row k0 + j / 4, columns m0 + 4 (j % 4), and lane i receives column m0 + i at rows k0 .. k0 + 3
// (so two reads give a lane its 8 k of one m).  The 32 lanes served per LDS cycle cover four
// rows x 64 bytes; the slot permutation spreads them over all 64 banks.  Rows at or past the
// operand's ``valid`` (the k extent) read as zero.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "rf_mfma.h"

namespace rf {

struct PipeOperand {
    const void* ptr;   // row 0 of the tile, k = 0
    int64_t ld;        // row stride in elements
    int64_t valid;     // rows of the tile that exist (rows >= valid read as zero)
};

// Work-group renumbering for L2 locality.  The dispatcher deals consecutive work-groups to
// the 8 XCDs in turn, and each XCD has its own L2.  ``xcd_order`` renumbers work-group b so
// that every XCD receives one contiguous range of the logical order; ``grouped_tile`` then
// walks a range in column groups of ``gf`` row tiles, so the 32 work-groups an XCD runs at
// once share a few operand tiles (gf row tiles x 32/gf column tiles).
__device__ inline int xcd_order(int b, int n) {
    constexpr int kXcd = 8;
    const int q = n / kXcd, r = n % kXcd;
    const int x = b % kXcd, i = b / kXcd;
    return x * q + (x < r ? x : r) + i;
}
__device__ inline void grouped_tile(int v, int n_rows, int n_cols, int gf, int& row, int& col) {
    const int span = gf * n_cols;
    const int grp = v / span;
    const int f0 = grp * gf;
    const int gs = (n_rows - f0) < gf ? (n_rows - f0) : gf;
    const int w = v - grp * span;
    row = f0 + w % gs;
    col = w / gs;
}

// A tile order for launches whose row tiles have unequal K lengths (longer for lower rows):
// logical index l (after xcd_order, so each XCD receives one contiguous range) walks the n_cols
// columns in 8 blocks of ceil(n_cols / 8), one per XCD range when n_cols divides by 8; within a
// block, row tiles in groups of 4 go slowest (longest first), then the block's columns, then
// the 4 rows of the group.  Every XCD so gets the same mix of long and short tiles, starts on
// its long ones, and runs 4 row tiles x 8 columns at a time.
__device__ inline void balanced_tile(int l, int n_rows, int n_cols, int& row, int& col) {
    const int cb = (n_cols + 7) / 8;
    const int blk = l / (n_rows * cb);
    const int r = l - blk * n_rows * cb;
    const int ck = (n_cols - blk * cb) < cb ? (n_cols - blk * cb) : cb;
    const int n_grp = (n_rows + 3) / 4;
    int grp = r / (4 * ck);
    if (grp > n_grp - 1) grp = n_grp - 1;
    const int w = r - grp * 4 * ck;
    const int gs = (n_rows - 4 * grp) < 4 ? (n_rows - 4 * grp) : 4;
    row = 4 * grp + w % gs;
    col = blk * cb + w / gs;
}

template <int WAVES, int NSETS = 2, bool MMAJOR = false>
struct PipeGemmW {
    static_assert(WAVES == 4 || WAVES == 8, "4 waves (one per SIMD) or 8 (two per SIMD)");
    static_assert(NSETS == 1 || NSETS == 2, "register sets of staged loads");
    static_assert(!MMAJOR || WAVES == 4, "M-major operands: four waves");
    static constexpr int kThr = WAVES * 64;
    static constexpr int BM = 256, BN = 256, BK = 64;
    static constexpr int ROWB = 128;                       // bytes of one row per k-step
    static constexpr int STAGE_BYTES = (BM + BN) * ROWB;   // 64 KiB
    static constexpr int LDS_BYTES = 2 * STAGE_BYTES;      // 128 KiB
    static constexpr int WGM = 2, WGN = WAVES / 2;         // wave grid
    static constexpr int WTM = BM / WGM, WTN = BN / WGN;   // wave tile: 128 x 128 or 128 x 64
    static constexpr int SM = WTM / 32, SN = WTN / 32;
    static constexpr int VA = BM * 8 / kThr;               // 16-byte vectors per thread per step
    static constexpr int VB = BN * 8 / kThr;
    static constexpr int ROWS_J = kThr / 8;                // rows between a thread's vectors
    static constexpr int NR = (MMAJOR ? 2 : 1) * (SM + SN);  // fragment reads per k-slice
    static constexpr int NM = SM * SN;                     // MFMAs per k-slice

    f32x16 acc[SM][SN];

    __device__ static inline __amdgpu_buffer_rsrc_t rsrc(const PipeOperand& op, int rows) {
        // byte range covers the rows that exist; a row at or past ``valid`` starts beyond it
        // (M-major: the rows are k, all of them counted)
        int64_t nrows = MMAJOR || op.valid < rows ? op.valid : rows;
        if (nrows < 0) nrows = 0;
        const int64_t bytes = nrows * op.ld * 2;
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(op.ptr), (short)0, (int)bytes, 0x00020000);
    }

    struct Regs {
        u32x4 a[VA], b[VB];
    };

    // Full K loop over ``nk`` k-steps; nk must be even (the loop is unrolled by two so that
    // the two register sets are addressed statically).  With a_fold > 0 (K-contiguous operands),
    // k-step kt of A is read from step kt - a_fold once kt reaches a_fold: A's first a_fold
    // steps serve twice.
    __device__ inline void run(char* lds, const PipeOperand& A, const PipeOperand& B, int nk, int a_fold = 0) {
        const int t = threadIdx.x;
        const int lane = t & 63;
        const int wave = t >> 6;
        const int wm = wave / WGN, wn = wave % WGN;

#pragma unroll
        for (int i = 0; i < SM; ++i)
#pragma unroll
            for (int j = 0; j < SN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
        if (nk <= 0) return;

        const __amdgpu_buffer_rsrc_t ra = rsrc(A, BM);
        const __amdgpu_buffer_rsrc_t rb = rsrc(B, BN);
        // global: row (t >> 3) + ROWS_J j, logical chunk t & 7 (M-major: row (t >> 5) + 8 j of
        // the k-step, chunk t & 31)
        const int gA = MMAJOR ? (int)((t >> 5) * A.ld * 2) + (t & 31) * 16 : (int)((t >> 3) * A.ld * 2) + (t & 7) * 16;
        const int gB = MMAJOR ? (int)((t >> 5) * B.ld * 2) + (t & 31) * 16 : (int)((t >> 3) * B.ld * 2) + (t & 7) * 16;
        const int strideA = (int)((MMAJOR ? 8 : ROWS_J) * A.ld * 2);
        const int strideB = (int)((MMAJOR ? 8 : ROWS_J) * B.ld * 2);
        // LDS write slot: row (t >> 3) + ROWS_J j has (row >> 1) & 7 == (t >> 4) & 7 (M-major:
        // 512-byte rows (t >> 5) + 8 j, whose k & 3 is (t >> 5) & 3; stride 4096 bytes)
        const int wofs = MMAJOR ? (t >> 5) * 512 + (((t & 31) ^ (4 * ((t >> 5) & 3))) << 4)
                                : (t >> 3) * ROWB + (((t & 7) ^ ((t >> 4) & 7)) << 4);
        const int wstep = MMAJOR ? 4096 : ROWS_J * ROWB;
        // LDS fragment reads: row (lane & 31) of a 32-row block, chunk 2 kk + (lane >> 5)
        const int rA = (wm * WTM + (lane & 31)) * ROWB;
        const int rB = (BM + wn * WTN + (lane & 31)) * ROWB;
        int cofs[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) cofs[kk] = ((2 * kk + (lane >> 5)) ^ ((lane >> 1) & 7)) << 4;

        // k-step offsets: K-major steps move along the row (buffer offset), M-major steps move
        // down 64 rows, kept in the range-checked vector offset so rows past the end read zero
        auto gload_a = [&](Regs& g, int kt) {
            int kc = kt < nk ? kt : nk - 1;
            if (a_fold > 0 && kc >= a_fold) kc -= a_fold;
            const int kb = MMAJOR ? 0 : kc * ROWB;
            const int kv = MMAJOR ? (int)(kc * 64 * A.ld * 2) : 0;
#pragma unroll
            for (int j = 0; j < VA; ++j) g.a[j] = __builtin_amdgcn_raw_buffer_load_b128(ra, gA + kv + j * strideA, kb, 0);
        };
        auto gload_b = [&](Regs& g, int kt) {
            const int kc = kt < nk ? kt : nk - 1;
            const int kb = MMAJOR ? 0 : kc * ROWB;
            const int kv = MMAJOR ? (int)(kc * 64 * B.ld * 2) : 0;
#pragma unroll
            for (int j = 0; j < VB; ++j) g.b[j] = __builtin_amdgcn_raw_buffer_load_b128(rb, gB + kv + j * strideB, kb, 0);
        };
        auto swrite_a = [&](const Regs& g, char* st) {
#pragma unroll
            for (int j = 0; j < VA; ++j) *(u32x4*)(st + wofs + j * wstep) = g.a[j];
        };
        auto swrite_b = [&](const Regs& g, char* st) {
#pragma unroll
            for (int j = 0; j < VB; ++j) *(u32x4*)(st + BM * ROWB + wofs + j * wstep) = g.b[j];
        };
        u32x4 fa[2][SM], fb[2][SN];
        // M-major fragments: lane l = 16 g + j reads row kk * 16 + 8 (g >> 1) + 4 h + (j >> 2),
        // columns (g & 1) * 16 + 4 (j & 3) of its 32-column block, for h = 0, 1
        const int tk = ((lane >> 5) << 3) + ((lane & 15) >> 2);
        const int tm = (((lane >> 4) & 1) << 4) + 4 * (lane & 3);
        auto tread = [&](const char* base, int k, int m) -> uint2 {
            typedef short v4i16 __attribute__((ext_vector_type(4)));
            typedef __attribute__((address_space(3))) v4i16 lds_v4;
            const int off = k * 512 + ((((m >> 3) ^ (4 * (k & 3))) << 4) | ((m & 7) * 2));
            const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_v4*)((__attribute__((address_space(3))) char*)base + off));
            return __builtin_bit_cast(uint2, v);
        };
        auto fread = [&](int buf, const char* st, int kk) {
            if constexpr (MMAJOR) {
#pragma unroll
                for (int i = 0; i < SM; ++i) {
                    const uint2 lo = tread(st, kk * 16 + tk, wm * WTM + i * 32 + tm);
                    const uint2 hi = tread(st, kk * 16 + 4 + tk, wm * WTM + i * 32 + tm);
                    fa[buf][i] = u32x4{lo.x, lo.y, hi.x, hi.y};
                }
#pragma unroll
                for (int j = 0; j < SN; ++j) {
                    const uint2 lo = tread(st + BM * ROWB, kk * 16 + tk, wn * WTN + j * 32 + tm);
                    const uint2 hi = tread(st + BM * ROWB, kk * 16 + 4 + tk, wn * WTN + j * 32 + tm);
                    fb[buf][j] = u32x4{lo.x, lo.y, hi.x, hi.y};
                }
            } else {
#pragma unroll
                for (int i = 0; i < SM; ++i) fa[buf][i] = *(const u32x4*)(st + rA + i * 32 * ROWB + cofs[kk]);
#pragma unroll
                for (int j = 0; j < SN; ++j) fb[buf][j] = *(const u32x4*)(st + rB + j * 32 * ROWB + cofs[kk]);
            }
        };
        auto mfma = [&](int buf, int i0, int i1) {
#pragma unroll
            for (int i = i0; i < i1; ++i)
#pragma unroll
                for (int j = 0; j < SN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, fa[buf][i]),
                                                                       __builtin_bit_cast(bf16x8, fb[buf][j]),
                                                                       acc[i][j], 0, 0, 0);
        };
        // Group barriers (mask 0x008 MFMA, 0x100 LDS read, 0x200 LDS write, 0x020 VMEM read).
        // A slice with a stage half to write: VA groups of {read, MFMA, write, load, MFMA}, then
        // the remaining reads and MFMAs.  A slice without: {read, MFMA} pairs, then the rest.
        auto sched_write_slice = [&]() {
#pragma unroll
            for (int i = 0; i < VA; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            }
            if constexpr (NR > VA) __builtin_amdgcn_sched_group_barrier(0x100, NR - VA, 0);
            if constexpr (NM > 2 * VA) __builtin_amdgcn_sched_group_barrier(0x008, NM - 2 * VA, 0);
        };
        auto sched_read_slice = [&](auto n_mfma_c) {
            constexpr int n_mfma = decltype(n_mfma_c)::value;
            constexpr int pairs = NR < n_mfma ? NR : n_mfma;
#pragma unroll
            for (int i = 0; i < pairs; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            }
            if constexpr (NR > pairs) __builtin_amdgcn_sched_group_barrier(0x100, NR - pairs, 0);
            if constexpr (n_mfma > pairs) __builtin_amdgcn_sched_group_barrier(0x008, n_mfma - pairs, 0);
        };

        // One k-step.  ``g`` holds step kt+1 (written to the other LDS stage here) and is then
        // refilled with step kt+1+NSETS.  Each slice is its own scheduling region.
        auto step = [&](int kt, Regs& g) {
            char* cur = lds + (kt & 1) * STAGE_BYTES;
            char* nxt = lds + ((kt + 1) & 1) * STAGE_BYTES;
            // slice 0: next slice's fragments, A half of the next stage, its refill
            fread(1, cur, 1);
            swrite_a(g, nxt);
            gload_a(g, kt + 1 + NSETS);
            mfma(0, 0, SM);
            sched_write_slice();
            __builtin_amdgcn_sched_barrier(0);
            // slice 1: fragments, B half of the next stage, its refill
            fread(0, cur, 2);
            swrite_b(g, nxt);
            gload_b(g, kt + 1 + NSETS);
            mfma(1, 0, SM);
            sched_write_slice();
            __builtin_amdgcn_sched_barrier(0);
            // slice 2
            fread(1, cur, 3);
            mfma(0, 0, SM);
            sched_read_slice(std::integral_constant<int, NM>{});
            __builtin_amdgcn_sched_barrier(0);
            // slice 3: half, barrier, first fragments of the next stage, other half
            mfma(1, 0, SM / 2);
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();
            fread(0, nxt, 0);
            mfma(1, SM / 2, SM);
            sched_read_slice(std::integral_constant<int, NM / 2>{});
            __builtin_amdgcn_sched_barrier(0);
        };

        // prologue: step 0 in LDS stage 0, the next NSETS steps in flight to the register sets
        // (fences keep the loads in step order, which the in-order load counter relies on)
        if constexpr (NSETS == 2) {
            Regs g0, g1;
            gload_a(g0, 0);
            gload_b(g0, 0);
            __builtin_amdgcn_sched_barrier(0);
            gload_a(g1, 1);
            gload_b(g1, 1);
            __builtin_amdgcn_sched_barrier(0);
            swrite_a(g0, lds);
            swrite_b(g0, lds);
            __builtin_amdgcn_sched_barrier(0);
            gload_a(g0, 2);
            __builtin_amdgcn_sched_barrier(0);
            gload_b(g0, 2);
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();
            fread(0, lds, 0);
            for (int kt = 0; kt < nk; kt += 2) {
                step(kt, g1);       // writes step kt+1 (odd), refills with kt+3
                step(kt + 1, g0);   // writes step kt+2 (even), refills with kt+4
            }
        } else {
            Regs g;
            gload_a(g, 0);
            gload_b(g, 0);
            __builtin_amdgcn_sched_barrier(0);
            swrite_a(g, lds);
            swrite_b(g, lds);
            __builtin_amdgcn_sched_barrier(0);
            gload_a(g, 1);
            __builtin_amdgcn_sched_barrier(0);
            gload_b(g, 1);
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();
            fread(0, lds, 0);
            for (int kt = 0; kt < nk; ++kt) step(kt, g);   // writes step kt+1, refills with kt+2
        }
        // the last fragment reads and stage writes target LDS the caller may reuse
        __syncthreads();
    }

    // Coordinates of accumulator register r of block (i, j) for this lane, relative to the
    // tile origin.
    __device__ static inline int row_of(int i, int r) {
        const int lane = threadIdx.x & 63, wm = (threadIdx.x >> 6) / WGN;
        return wm * WTM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
    }
    __device__ static inline int col_of(int j) {
        const int lane = threadIdx.x & 63, wn = (threadIdx.x >> 6) % WGN;
        return wn * WTN + j * 32 + (lane & 31);
    }
};

// Variant with a pre-packed A operand (weights) for the fill's products.
//
// The four waves are stacked along m: wave w computes rows 64 w .. 64 w + 63 of the 256 x 256
// tile against all 256 columns (2 x 8 blocks of v_mfma_f32_32x32x16_bf16, 256 accumulation
// registers).  A wave's A rows belong to it alone, so A skips LDS: it is stored pre-packed in
// fragment order (rf_pack_weights) and every fragment is one 1 KiB contiguous load straight
// into registers, issued two k-steps ahead.  Only B is staged through LDS as in PipeGemmW,
// which halves the LDS stage writes per k-step (the data movement that lowers the
// power-limited clock most).
//
// Packed A, one 256-row tile of K columns: element (r, k) sits at element offset
//   (k / 64) * 16384 + (r / 64) * 4096 + ((k % 64) / 16) * 1024 + ((r % 64) / 32) * 512
//   + (((k % 16) / 8) * 32 + r % 32) * 8 + k % 8,
// i.e. k-step, wave, k-slice, block, then the 64 lanes' 16-byte fragments.
// Eight int8 codes (byte e of the pair of words = element e) as eight bf16 values: each code
// sign-extended, converted to fp32 and cut to its upper half, which is exact for |code| <= 127.
__device__ inline bf16x8 i8x8_to_bf16x8(u32x2 v) {
    u32x4 r;
#pragma unroll
    for (int w = 0; w < 2; ++w)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const float f0 = (float)((int)(v[w] << (24 - 16 * h)) >> 24);
            const float f1 = (float)((int)(v[w] << (16 - 16 * h)) >> 24);
            r[2 * w + h] = (__builtin_bit_cast(uint32_t, f1) & 0xffff0000u) | (__builtin_bit_cast(uint32_t, f0) >> 16);
        }
    return __builtin_bit_cast(bf16x8, r);
}

struct PackedAGemm {
    static constexpr int kThr = 256;
    static constexpr int BM = 256, BN = 256, BK = 64;
    static constexpr int ROWB = 128;                       // bytes of one B row per k-step
    static constexpr int STAGE_BYTES = BN * ROWB;          // 32 KiB
    static constexpr int LDS_BYTES = 2 * STAGE_BYTES;
    static constexpr int WGM = 4, WGN = 1;
    static constexpr int WTM = 64, WTN = 256;
    static constexpr int SM = 2, SN = 8;
    static constexpr int VB = BN * 8 / kThr;               // 16-byte vectors per thread per step
    static constexpr int ROWS_J = kThr / 8;                // rows between a thread's vectors
    static constexpr int kStepBytes = BM * BK * 2;         // packed A bytes per k-step

    f32x16 acc[SM][SN];

    struct Regs {
        u32x4 b[VB];
    };

    // Full K loop over ``nk`` k-steps (even).  A.ptr is the packed tile; A.ld and A.valid are
    // unused (a packed tile always holds 256 rows).  With FOLD, k-step kt of B is read from step
    // kt < b_fold ? kt : kt - b_fold of its rows (B's first b_fold steps serve twice).  With SEG,
    // the K loop visits segments of 4 k-steps (256 columns) seg_stride steps apart: logical step
    // kt reads step (kt / 4) * seg_stride + kt % 4 of both operands.  With REV the K loop runs
    // from the last step down (logical step kt reads step nk - 1 - kt), so tiles of different
    // lengths that end at the same column read the same columns at the same time.  With I8 the
    // packed tile holds int8 codes (the same element order, one byte each): each fragment is an
    // 8-byte load, widened to bf16 in registers (exact: |code| <= 127 needs 7 bits) just before
    // its MFMAs.
    template <bool FOLD = false, bool SEG = false, bool REV = false, bool I8 = false>
    __device__ inline void run(char* lds, const PipeOperand& A, const PipeOperand& B, int nk, int b_fold = 0,
                               int seg_stride = 4) {
        static_assert(!(REV && (FOLD || SEG)), "a reversed K loop reads plain steps");
        constexpr int AB = I8 ? 1 : 2;   // bytes per A element
        const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
#pragma unroll
        for (int i = 0; i < SM; ++i)
#pragma unroll
            for (int j = 0; j < SN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
        if (nk <= 0) return;
        // physical k-step of logical step kc (uniform by construction, said so for the compiler)
        auto phys = [&](int kc) {
            if constexpr (SEG) return __builtin_amdgcn_readfirstlane((kc >> 2) * seg_stride + (kc & 3));
            if constexpr (REV) return __builtin_amdgcn_readfirstlane(nk - 1 - kc);
            return kc;
        };
        const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<void*>(A.ptr), (short)0, ((REV ? nk - 1 : phys(nk - 1)) + 1) * (kStepBytes / 2 * AB), 0x00020000);
        int64_t nb = B.valid < BN ? B.valid : BN;
        if (nb < 0) nb = 0;
        const __amdgpu_buffer_rsrc_t rb =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(B.ptr), (short)0, (int)(nb * B.ld * 2), 0x00020000);
        // B staging as in PipeGemmW: row (t >> 3) + 32 j, logical chunk t & 7, slot
        // chunk ^ ((row >> 1) & 7)
        const int gB = (int)((t >> 3) * B.ld * 2) + (t & 7) * 16;
        const int strideB = (int)(ROWS_J * B.ld * 2);
        const int wofs = (t >> 3) * ROWB + (((t & 7) ^ ((t >> 4) & 7)) << 4);
        const int wstep = ROWS_J * ROWB;
        const int rB = (lane & 31) * ROWB;
        int cofs[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) cofs[kk] = ((2 * kk + (lane >> 5)) ^ ((lane >> 1) & 7)) << 4;
        // the wave offset stays in the vector offset: a scalar offset must be provably uniform
        const int av = (wave * 8192 + lane * 16) / 2 * AB;

        // A fragments of two k-steps (parity p), 4 slices x 2 blocks each
        using AFrag = std::conditional_t<I8, u32x2, u32x4>;
        AFrag fa[2][4][SM];
        auto aload = [&](int p, int kk, int kt) {
            const int kc = phys(kt < nk ? kt : nk - 1);
#pragma unroll
            for (int i = 0; i < SM; ++i) {
                if constexpr (I8)
                    fa[p][kk][i] = __builtin_amdgcn_raw_buffer_load_b64(ra, av, kc * (kStepBytes / 2) + (kk * 2 + i) * 512, 0);
                else
                    fa[p][kk][i] = __builtin_amdgcn_raw_buffer_load_b128(ra, av, kc * kStepBytes + (kk * 2 + i) * 1024, 0);
            }
        };
        auto afrag = [&](int p, int kk, int i) -> bf16x8 {
            if constexpr (I8) return i8x8_to_bf16x8(fa[p][kk][i]);
            else return __builtin_bit_cast(bf16x8, fa[p][kk][i]);
        };
        auto gload_b = [&](Regs& g, int kt, int j0, int j1) {
            int kc = kt < nk ? kt : nk - 1;
            if constexpr (FOLD) {
                if (kc >= b_fold) kc -= b_fold;
                // uniform by construction; said so, or the compiler wraps each load in a
                // waterfall loop
                kc = __builtin_amdgcn_readfirstlane(kc);
            }
            kc = phys(kc);
#pragma unroll
            for (int j = j0; j < j1; ++j) g.b[j] = __builtin_amdgcn_raw_buffer_load_b128(rb, gB + j * strideB, kc * ROWB, 0);
        };
        auto swrite_b = [&](const Regs& g, char* st, int j0, int j1) {
#pragma unroll
            for (int j = j0; j < j1; ++j) *(u32x4*)(st + wofs + j * wstep) = g.b[j];
        };
        u32x4 fb[2][SN];
        auto fread = [&](int buf, const char* st, int kk) {
#pragma unroll
            for (int j = 0; j < SN; ++j) fb[buf][j] = *(const u32x4*)(st + rB + j * 32 * ROWB + cofs[kk]);
        };
        auto mfma = [&](int buf, int p, int kk, int j0, int j1) {
            bf16x8 a[SM];
#pragma unroll
            for (int i = 0; i < SM; ++i) a[i] = afrag(p, kk, i);
#pragma unroll
            for (int j = j0; j < j1; ++j)
#pragma unroll
                for (int i = 0; i < SM; ++i)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], __builtin_bit_cast(bf16x8, fb[buf][j]),
                                                                       acc[i][j], 0, 0, 0);
        };
        // group barriers (mask 0x008 MFMA, 0x100 LDS read, 0x200 LDS write, 0x020 VMEM read)
        auto sched_write_slice = [&]() {
#pragma unroll
            for (int i = 0; i < VB / 2; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x100, SN - VB / 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, SM, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        };
        auto sched_read_slice = [&]() {
#pragma unroll
            for (int i = 0; i < SN; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, SM, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        };
        // One k-step: ``g`` holds B of step kt+1 (written to the other stage here, half in each
        // of the first two slices) and is refilled with step kt+3; each slice's A fragments are
        // reloaded with step kt+2 once its MFMAs have read them.
        auto step = [&](int kt, Regs& g, auto par) {
            constexpr int P = decltype(par)::value;
            char* cur = lds + P * STAGE_BYTES;
            char* nxt = lds + (1 - P) * STAGE_BYTES;
            fread(1, cur, 1);
            swrite_b(g, nxt, 0, VB / 2);
            gload_b(g, kt + 3, 0, VB / 2);
            mfma(0, P, 0, 0, SN);
            aload(P, 0, kt + 2);
            sched_write_slice();
            __builtin_amdgcn_sched_barrier(0);
            fread(0, cur, 2);
            swrite_b(g, nxt, VB / 2, VB);
            gload_b(g, kt + 3, VB / 2, VB);
            mfma(1, P, 1, 0, SN);
            aload(P, 1, kt + 2);
            sched_write_slice();
            __builtin_amdgcn_sched_barrier(0);
            fread(1, cur, 3);
            mfma(0, P, 2, 0, SN);
            aload(P, 2, kt + 2);
            sched_read_slice();
            __builtin_amdgcn_sched_barrier(0);
            // last slice: half, barrier, first fragments of the next stage, other half
            mfma(1, P, 3, 0, SN / 2);
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();
            fread(0, nxt, 0);
            mfma(1, P, 3, SN / 2, SN);
            aload(P, 3, kt + 2);
            __builtin_amdgcn_sched_barrier(0);
        };
        // prologue: A of steps 0 and 1, B of step 0 in stage 0, B of steps 1 and 2 in flight
        // (fences keep the loads in step order, which the in-order load counter relies on)
        Regs g0, g1;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) aload(0, kk, 0);
        gload_b(g0, 0, 0, VB);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) aload(1, kk, 1);
        gload_b(g1, 1, 0, VB);
        __builtin_amdgcn_sched_barrier(0);
        swrite_b(g0, lds, 0, VB);
        __builtin_amdgcn_sched_barrier(0);
        gload_b(g0, 2, 0, VB);
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        fread(0, lds, 0);
        for (int kt = 0; kt < nk; kt += 2) {
            step(kt, g1, std::integral_constant<int, 0>{});       // writes B of kt+1, refills kt+3
            step(kt + 1, g0, std::integral_constant<int, 1>{});   // writes B of kt+2, refills kt+4
        }
        // the last fragment reads and stage writes target LDS the caller may reuse
        __syncthreads();
    }

    __device__ static inline int row_of(int i, int r) {
        const int lane = threadIdx.x & 63, wm = threadIdx.x >> 6;
        return wm * WTM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
    }
    __device__ static inline int col_of(int j) { return j * 32 + (threadIdx.x & 31); }
};

// Element offset of (r, k) of a packed matrix with K columns: 256-row tiles one after the
// other, each laid out as above.  The offset splits into the tile's base, a part of the row in
// the tile and a part of the column (both below 2^31 for K <= 65536).
__host__ __device__ inline int packed_row_part(int rt) {   // rt in [0, 256)
    return ((rt >> 6) << 12) + (((rt & 63) >> 5) << 9) + ((rt & 31) << 3);
}
__host__ __device__ inline int packed_col_part(int k) {
    return ((k >> 6) << 14) + (((k & 63) >> 4) << 10) + (((k & 15) >> 3) << 8) + (k & 7);
}
__host__ __device__ inline int64_t packed_index(int64_t r, int k, int64_t K) {
    return (r >> 8) * 256 * K + packed_row_part((int)(r & 255)) + packed_col_part(k);
}

// Source row, within its 256-row tile, of packed row p.  hd == 0 keeps the order; otherwise
// wave w's block i takes rows of pairs (f, f + hd/2) of the tile's heads: pair q = 32 w + r % 32,
// first partner in block 0, second in block 1, so a RoPE pair meets in one lane's registers.
__host__ __device__ inline int packed_source_row(int p, int hd) {
    if (hd == 0) return p;
    const int half = hd >> 1;
    const int q = ((p >> 6) << 5) + (p & 31);
    return (q / half) * hd + q % half + ((p >> 5) & 1) * half;
}

// One wave per SIMD with two load sets measured best on the fill and Gram products; two waves
// per SIMD (PipeGemmW<8, 1>, one load set to fit 256 registers per wave) measured equal.
using PipeGemm = PipeGemmW<4, 2>;
constexpr int kPipeThreads = PipeGemm::kThr;

}  // namespace rf
