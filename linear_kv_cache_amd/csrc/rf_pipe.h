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

template <int WAVES, int NSETS = 2>
struct PipeGemmW {
    static_assert(WAVES == 4 || WAVES == 8, "4 waves (one per SIMD) or 8 (two per SIMD)");
    static_assert(NSETS == 1 || NSETS == 2, "register sets of staged loads");
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
    static constexpr int NR = SM + SN;                     // fragment reads per k-slice
    static constexpr int NM = SM * SN;                     // MFMAs per k-slice

    f32x16 acc[SM][SN];

    __device__ static inline __amdgpu_buffer_rsrc_t rsrc(const PipeOperand& op, int rows) {
        // byte range covers the rows that exist; a row at or past ``valid`` starts beyond it
        int64_t nrows = op.valid < rows ? op.valid : rows;
        if (nrows < 0) nrows = 0;
        const int64_t bytes = nrows * op.ld * 2;
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(op.ptr), (short)0, (int)bytes, 0x00020000);
    }

    struct Regs {
        u32x4 a[VA], b[VB];
    };

    // Full K loop over ``nk`` k-steps; nk must be even (the loop is unrolled by two so that
    // the two register sets are addressed statically).
    __device__ inline void run(char* lds, const PipeOperand& A, const PipeOperand& B, int nk) {
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
        // global: row (t >> 3) + ROWS_J j, logical chunk t & 7
        const int gA = (int)((t >> 3) * A.ld * 2) + (t & 7) * 16;
        const int gB = (int)((t >> 3) * B.ld * 2) + (t & 7) * 16;
        const int strideA = (int)(ROWS_J * A.ld * 2);
        const int strideB = (int)(ROWS_J * B.ld * 2);
        // LDS write slot: row (t >> 3) + ROWS_J j has (row >> 1) & 7 == (t >> 4) & 7
        const int wofs = (t >> 3) * ROWB + (((t & 7) ^ ((t >> 4) & 7)) << 4);
        // LDS fragment reads: row (lane & 31) of a 32-row block, chunk 2 kk + (lane >> 5)
        const int rA = (wm * WTM + (lane & 31)) * ROWB;
        const int rB = (BM + wn * WTN + (lane & 31)) * ROWB;
        int cofs[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) cofs[kk] = ((2 * kk + (lane >> 5)) ^ ((lane >> 1) & 7)) << 4;

        auto gload_a = [&](Regs& g, int kt) {
            const int kb = (kt < nk ? kt : nk - 1) * ROWB;
#pragma unroll
            for (int j = 0; j < VA; ++j) g.a[j] = __builtin_amdgcn_raw_buffer_load_b128(ra, gA + j * strideA, kb, 0);
        };
        auto gload_b = [&](Regs& g, int kt) {
            const int kb = (kt < nk ? kt : nk - 1) * ROWB;
#pragma unroll
            for (int j = 0; j < VB; ++j) g.b[j] = __builtin_amdgcn_raw_buffer_load_b128(rb, gB + j * strideB, kb, 0);
        };
        auto swrite_a = [&](const Regs& g, char* st) {
#pragma unroll
            for (int j = 0; j < VA; ++j) *(u32x4*)(st + wofs + j * ROWS_J * ROWB) = g.a[j];
        };
        auto swrite_b = [&](const Regs& g, char* st) {
#pragma unroll
            for (int j = 0; j < VB; ++j) *(u32x4*)(st + BM * ROWB + wofs + j * ROWS_J * ROWB) = g.b[j];
        };
        u32x4 fa[2][SM], fb[2][SN];
        auto fread = [&](int buf, const char* st, int kk) {
#pragma unroll
            for (int i = 0; i < SM; ++i) fa[buf][i] = *(const u32x4*)(st + rA + i * 32 * ROWB + cofs[kk]);
#pragma unroll
            for (int j = 0; j < SN; ++j) fb[buf][j] = *(const u32x4*)(st + rB + j * 32 * ROWB + cofs[kk]);
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

// ---------------------------------------------------------------------------------------------
// The same 256 x 256 tile (4 waves, 2 x 2 grid, 128 x 128 per wave, v_mfma_f32_32x32x16_bf16),
// fed by direct global -> LDS loads (buffer_load_dwordx4 ... lds): no staging registers and no
// LDS write instructions.
//   k-steps of 32 elements (64 bytes per operand row); four LDS stages of 32 KiB in a ring;
//   the loads of step kt+3 are issued during step kt, so each has about three steps to land.
//   One load instruction fills 1 KiB of LDS: 16 rows x 64 bytes; lane l supplies row l / 4 and
//   the 16-byte slot l % 4, into which it loads logical chunk (l % 4) ^ ((row >> 2) & 3).  With
//   64 banks, the 16 rows read by 16 lanes for one logical chunk then hit 16 distinct bank
//   groups.
//   Completion is tracked by hand: before the barrier that publishes step kt+1, each wave waits
//   until at most 16 of its loads (those of steps kt+2 and kt+3) are outstanding.  Loads of
//   steps past the end use an empty buffer range and move no data.
struct DmaGemm {
    static constexpr int kThr = 256;
    static constexpr int BM = 256, BN = 256, BK = 32;
    static constexpr int ROWB = 64;                        // bytes of one row per k-step
    static constexpr int STAGE_BYTES = (BM + BN) * ROWB;   // 32 KiB
    static constexpr int NSTAGE = 4;
    static constexpr int LDS_BYTES = NSTAGE * STAGE_BYTES; // 128 KiB
    static constexpr int WGM = 2, WGN = 2;
    static constexpr int WTM = BM / WGM, WTN = BN / WGN;   // 128 x 128 per wave
    static constexpr int SM = WTM / 32, SN = WTN / 32;
    static constexpr int NI = BM * ROWB / 1024 / 4;       // load instructions per wave per operand per step

    f32x16 acc[SM][SN];

    __device__ static inline __amdgpu_buffer_rsrc_t rsrc(const PipeOperand& op, int rows) {
        int64_t nrows = op.valid < rows ? op.valid : rows;
        if (nrows < 0) nrows = 0;
        const int64_t bytes = nrows * op.ld * 2;
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(op.ptr), (short)0, (int)bytes, 0x00020000);
    }

    __device__ inline void run(char* lds, const PipeOperand& A, const PipeOperand& B, int nk) {
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
        const __amdgpu_buffer_rsrc_t rnone = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(A.ptr), (short)0, 0, 0x00020000);
        const int wu = __builtin_amdgcn_readfirstlane(wave);
        // load instruction j of this wave covers rows (wave * NI + j) * 16 .. + 16 of an operand
        const int lrow = lane >> 2;
        const int lchunk = (lane & 3) ^ ((lane >> 4) & 3);
        const int vA = (int)((wave * NI * 16 + lrow) * A.ld * 2) + lchunk * 16;
        const int vB = (int)((wave * NI * 16 + lrow) * B.ld * 2) + lchunk * 16;
        const int jA = (int)(16 * A.ld * 2), jB = (int)(16 * B.ld * 2);
        // fragment reads: row (lane & 31) of a 32-row block, chunk 2 kk + (lane >> 5)
        const int rA = (wm * WTM + (lane & 31)) * ROWB;
        const int rB = (BM + wn * WTN + (lane & 31)) * ROWB;
        int cofs[2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) cofs[kk] = ((2 * kk + (lane >> 5)) ^ ((lane >> 2) & 3)) << 4;

        typedef __attribute__((address_space(3))) void* lds_ptr_t;
        auto dma = [&](int kt) {
            char* st = lds + (kt & (NSTAGE - 1)) * STAGE_BYTES;
            const bool live = kt < nk;
            const __amdgpu_buffer_rsrc_t a_ = live ? ra : rnone;
            const __amdgpu_buffer_rsrc_t b_ = live ? rb : rnone;
            const int ko = kt * ROWB;
#pragma unroll
            for (int j = 0; j < NI; ++j)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(a_, (lds_ptr_t)(st + (wu * NI + j) * 1024), 16, vA,
                                                         ko + j * jA, 0, 0);
#pragma unroll
            for (int j = 0; j < NI; ++j)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(b_, (lds_ptr_t)(st + BM * ROWB + (wu * NI + j) * 1024), 16,
                                                         vB, ko + j * jB, 0, 0);
        };
        u32x4 fa[2][SM], fb[2][SN];
        auto fread = [&](int buf, const char* st, int kk) {
#pragma unroll
            for (int i = 0; i < SM; ++i) fa[buf][i] = *(const u32x4*)(st + rA + i * 32 * ROWB + cofs[kk]);
#pragma unroll
            for (int j = 0; j < SN; ++j) fb[buf][j] = *(const u32x4*)(st + rB + j * 32 * ROWB + cofs[kk]);
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
        // this wave's loads of the next step have landed and its fragment reads are done; then
        // every wave's (barrier without a memory fence: the waits are explicit)
        auto publish = [&]() {
            asm volatile("s_waitcnt vmcnt(16) lgkmcnt(0)" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        };

        // prologue: steps 0..2 in flight; wait for step 0
        dma(0);
        dma(1);
        dma(2);
        publish();
        fread(0, lds, 0);
        for (int kt = 0; kt < nk; ++kt) {
            const char* cur = lds + (kt & (NSTAGE - 1)) * STAGE_BYTES;
            const char* nxt = lds + ((kt + 1) & (NSTAGE - 1)) * STAGE_BYTES;
            // slice 0: second slice's fragments and the loads of step kt+3
            fread(1, cur, 1);
            dma(kt + 3);
            mfma(0, 0, SM);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
            // slice 1: half, publish step kt+1, its first fragments, other half
            mfma(1, 0, SM / 2);
            __builtin_amdgcn_sched_barrier(0);
            publish();
            fread(0, nxt, 0);
            mfma(1, SM / 2, SM);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // drain the loads past the end and let the caller reuse LDS
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        __syncthreads();
    }

    __device__ static inline int row_of(int i, int r) {
        const int lane = threadIdx.x & 63, wm = (threadIdx.x >> 6) / WGN;
        return wm * WTM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
    }
    __device__ static inline int col_of(int j) {
        const int lane = threadIdx.x & 63, wn = (threadIdx.x >> 6) % WGN;
        return wn * WTN + j * 32 + (lane & 31);
    }
};

// The same core with 64-element k-steps (whole 128-byte rows) and two LDS stages of 64 KiB:
// the loads of step kt+1 are issued at the start of step kt (right after the barrier that
// retires step kt-1's stage) and waited for at its end.  One load instruction fills 8 rows x
// 128 bytes; lane l supplies row l / 8 and slot l % 8, into which it loads logical chunk
// (l % 8) ^ ((row >> 1) & 7), the same swizzle as the register-staged core.
struct DmaGemm64 {
    static constexpr int kThr = 256;
    static constexpr int BM = 256, BN = 256, BK = 64;
    static constexpr int ROWB = 128;
    static constexpr int STAGE_BYTES = (BM + BN) * ROWB;   // 64 KiB
    static constexpr int LDS_BYTES = 2 * STAGE_BYTES;      // 128 KiB
    static constexpr int WGM = 2, WGN = 2;
    static constexpr int WTM = BM / WGM, WTN = BN / WGN;
    static constexpr int SM = WTM / 32, SN = WTN / 32;
    static constexpr int NI = BM * ROWB / 1024 / 4;       // 8 load instructions per wave per operand

    f32x16 acc[SM][SN];

    __device__ static inline __amdgpu_buffer_rsrc_t rsrc(const PipeOperand& op, int rows) {
        int64_t nrows = op.valid < rows ? op.valid : rows;
        if (nrows < 0) nrows = 0;
        const int64_t bytes = nrows * op.ld * 2;
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(op.ptr), (short)0, (int)bytes, 0x00020000);
    }

    __device__ inline void run(char* lds, const PipeOperand& A, const PipeOperand& B, int nk) {
        const int t = threadIdx.x;
        const int lane = t & 63;
        const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
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
        const __amdgpu_buffer_rsrc_t rnone = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(A.ptr), (short)0, 0, 0x00020000);
        // load instruction j of this wave covers rows (wave * NI + j) * 8 .. + 8; (row >> 1) & 7
        // = 4 ((wave * NI + j) & 1) + (lane >> 4) & 3, and NI is even, so two chunk patterns
        const int lrow = lane >> 3;
        const int ch0 = (lane & 7) ^ ((lane >> 4) & 3);
        const int ch1 = (lane & 7) ^ (4 + ((lane >> 4) & 3));
        const int vA0 = (int)((wave * NI * 8 + lrow) * A.ld * 2) + ch0 * 16;
        const int vA1 = (int)((wave * NI * 8 + lrow) * A.ld * 2) + ch1 * 16;
        const int vB0 = (int)((wave * NI * 8 + lrow) * B.ld * 2) + ch0 * 16;
        const int vB1 = (int)((wave * NI * 8 + lrow) * B.ld * 2) + ch1 * 16;
        const int jA = (int)(8 * A.ld * 2), jB = (int)(8 * B.ld * 2);
        const int rA = (wm * WTM + (lane & 31)) * ROWB;
        const int rB = (BM + wn * WTN + (lane & 31)) * ROWB;
        int cofs[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) cofs[kk] = ((2 * kk + (lane >> 5)) ^ ((lane >> 1) & 7)) << 4;

        typedef __attribute__((address_space(3))) void* lds_ptr_t;
        auto dma_a = [&](int kt) {
            char* st = lds + (kt & 1) * STAGE_BYTES;
            const __amdgpu_buffer_rsrc_t r_ = kt < nk ? ra : rnone;
#pragma unroll
            for (int j = 0; j < NI; ++j)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(r_, (lds_ptr_t)(st + (wave * NI + j) * 1024), 16,
                                                         (j & 1) ? vA1 : vA0, kt * ROWB + j * jA, 0, 0);
        };
        auto dma_b = [&](int kt) {
            char* st = lds + (kt & 1) * STAGE_BYTES + BM * ROWB;
            const __amdgpu_buffer_rsrc_t r_ = kt < nk ? rb : rnone;
#pragma unroll
            for (int j = 0; j < NI; ++j)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(r_, (lds_ptr_t)(st + (wave * NI + j) * 1024), 16,
                                                         (j & 1) ? vB1 : vB0, kt * ROWB + j * jB, 0, 0);
        };
        u32x4 fa[2][SM], fb[2][SN];
        auto fread = [&](int buf, const char* st, int kk) {
#pragma unroll
            for (int i = 0; i < SM; ++i) fa[buf][i] = *(const u32x4*)(st + rA + i * 32 * ROWB + cofs[kk]);
#pragma unroll
            for (int j = 0; j < SN; ++j) fb[buf][j] = *(const u32x4*)(st + rB + j * 32 * ROWB + cofs[kk]);
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
        auto publish = [&]() {
            asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        };
        auto interleave_dma = [&]() {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            }
        };

        // prologue: step 0 landed, its first fragments read
        dma_a(0);
        dma_b(0);
        publish();
        fread(0, lds, 0);
        for (int kt = 0; kt < nk; ++kt) {
            const char* cur = lds + (kt & 1) * STAGE_BYTES;
            const char* nxt = lds + ((kt + 1) & 1) * STAGE_BYTES;
            // slices 0 and 1 carry the loads of step kt+1 (its stage was retired by the last
            // barrier)
            fread(1, cur, 1);
            dma_a(kt + 1);
            mfma(0, 0, SM);
            interleave_dma();
            __builtin_amdgcn_sched_barrier(0);
            fread(0, cur, 2);
            dma_b(kt + 1);
            mfma(1, 0, SM);
            interleave_dma();
            __builtin_amdgcn_sched_barrier(0);
            // slice 2
            fread(1, cur, 3);
            mfma(0, 0, SM);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
            __builtin_amdgcn_sched_barrier(0);
            // slice 3: half, publish step kt+1, its first fragments, other half
            mfma(1, 0, SM / 2);
            __builtin_amdgcn_sched_barrier(0);
            publish();
            fread(0, nxt, 0);
            mfma(1, SM / 2, SM);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        __syncthreads();
    }

    __device__ static inline int row_of(int i, int r) {
        const int lane = threadIdx.x & 63, wm = (threadIdx.x >> 6) / WGN;
        return wm * WTM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
    }
    __device__ static inline int col_of(int j) {
        const int lane = threadIdx.x & 63, wn = (threadIdx.x >> 6) % WGN;
        return wn * WTN + j * 32 + (lane & 31);
    }
};

#ifndef RF_PIPE_WAVES
#define RF_PIPE_WAVES 4
#endif
#if defined(RF_PIPE_DMA64)
using PipeGemm = DmaGemm64;
#elif defined(RF_PIPE_DMA)
using PipeGemm = DmaGemm;
#else
using PipeGemm = PipeGemmW<RF_PIPE_WAVES, RF_PIPE_WAVES == 4 ? 2 : 1>;
#endif
constexpr int kPipeThreads = PipeGemm::kThr;

}  // namespace rf
