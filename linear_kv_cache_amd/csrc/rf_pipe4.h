// The packed-weight MFMA core on 512-row x 128-token tiles, for gfx950 (the fill's K/V
// product).  It shares the packed weight layout, the operand descriptor and the helpers of the
// 256 x 256 core in rf_pipe.h.
#pragma once

#include "rf_pipe.h"

namespace rf {

// The packed-weight core on a 512-row x 128-token tile: each wave owns 128 weight rows (the
// two 64-row groups 2 (w % 2), 2 (w % 2) + 1 of packed 256-row tile w / 2, the same packed
// layout as above) against all 128 tokens, 4 x 4 blocks.  Against the 256 x 256 tile each
// B fragment read from LDS feeds 4 MFMAs instead of 2 and a k-step stages 16 KiB instead of
// 32: per k-step a CU moves 80 KiB through LDS instead of 160, for 64 instead of 32 KiB of
// weight loads (the weight rows of a tile are no longer shared by token blocks in one
// work-group, only through L2).  The same pipeline: register-staged token rows written a
// k-step ahead, weight fragments two k-steps ahead, one barrier per k-step.
struct PackedAGemm4 {
    static constexpr int kThr = 256;
    static constexpr int BM = 512, BN = 128, BK = 64;
    static constexpr int ROWB = 128;
    static constexpr int STAGE_BYTES = BN * ROWB;          // 16 KiB
    static constexpr int LDS_BYTES = 2 * STAGE_BYTES;
    static constexpr int SM = 4, SN = 4;
    static constexpr int VB = BN * 8 / kThr;               // 4
    static constexpr int ROWS_J = kThr / 8;                // 32
    static constexpr int kStepBytes = 256 * BK * 2;        // one packed 256-row tile per k-step

    f32x16 acc[SM][SN];

    struct Regs {
        u32x4 b[VB];
    };

    // A.ptr: the first of the two packed 256-row tiles, A.ld = K (the second tile starts
    // 256 K elements later); B as in PackedAGemm.  nk k-steps (even).
    __device__ inline void run(char* lds, const PipeOperand& A, const PipeOperand& B, int nk) {
        const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
#pragma unroll
        for (int i = 0; i < SM; ++i)
#pragma unroll
            for (int j = 0; j < SN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
        if (nk <= 0) return;
        const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<void*>(A.ptr), (short)0, (int)(2 * 256 * A.ld * 2), 0x00020000);
        int64_t nb = B.valid < BN ? B.valid : BN;
        if (nb < 0) nb = 0;
        const __amdgpu_buffer_rsrc_t rb =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(B.ptr), (short)0, (int)(nb * B.ld * 2), 0x00020000);
        const int gB = (int)((t >> 3) * B.ld * 2) + (t & 7) * 16;
        const int strideB = (int)(ROWS_J * B.ld * 2);
        const int wofs = (t >> 3) * ROWB + (((t & 7) ^ ((t >> 4) & 7)) << 4);
        const int wstep = ROWS_J * ROWB;
        const int rB = (lane & 31) * ROWB;
        int cofs[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) cofs[kk] = ((2 * kk + (lane >> 5)) ^ ((lane >> 1) & 7)) << 4;
        // wave w: packed tile w / 2, its 64-row groups 2 (w % 2) and 2 (w % 2) + 1
        const int av = (int)((wave >> 1) * 256 * A.ld * 2) + (wave & 1) * 16384 + lane * 16;
        u32x4 fa[2][4][SM];
        auto aload = [&](int p, int kk, int kt) {
            const int kc = kt < nk ? kt : nk - 1;
#pragma unroll
            for (int i = 0; i < SM; ++i)
                fa[p][kk][i] = __builtin_amdgcn_raw_buffer_load_b128(ra, av, kc * kStepBytes + (i >> 1) * 8192 +
                                                                                kk * 2048 + (i & 1) * 1024, 0);
        };
        auto gload_b = [&](Regs& g, int kt, int j0, int j1) {
            const int kc = kt < nk ? kt : nk - 1;
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
#pragma unroll
            for (int j = j0; j < j1; ++j)
#pragma unroll
                for (int i = 0; i < SM; ++i)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, fa[p][kk][i]),
                                                                       __builtin_bit_cast(bf16x8, fb[buf][j]),
                                                                       acc[i][j], 0, 0, 0);
        };
        auto sched_write_slice = [&]() {
#pragma unroll
            for (int i = 0; i < VB / 2; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
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
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, SM, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        };
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
            mfma(1, P, 3, 0, SN / 2);
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();
            fread(0, nxt, 0);
            mfma(1, P, 3, SN / 2, SN);
            aload(P, 3, kt + 2);
            __builtin_amdgcn_sched_barrier(0);
        };
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
            step(kt, g1, std::integral_constant<int, 0>{});
            step(kt + 1, g0, std::integral_constant<int, 1>{});
        }
        __syncthreads();
    }
};

}  // namespace rf
