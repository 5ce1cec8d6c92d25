// Pipelined bf16 MFMA GEMM for batches of many tokens: C[m][n] = sum_k A[m][k] * B[n][k].
//
// One workgroup of 4 waves computes a BM x BN tile (each wave (BM/2) x (BN/2) with
// v_mfma_f32_32x32x16_bf16).  K advances in stages of 64 columns.  Each stage's operands are
// copied straight from global memory into LDS with global_load_lds_dwordx4 (no register
// staging), NS stages deep, so the copies of the next NS-1 stages are in flight while one
// stage is multiplied; one barrier per stage.
//
// A copy instruction moves 1 KB: lane l writes LDS position l of the instruction's block, and
// the lane picks its global source so that
//   * a row-major operand block holds 8 rows x 128 bytes (a full cache line per row), with the
//     16-byte chunks of row r stored XOR-swizzled by (r & 7), which keeps fragment reads free of
//     bank conflicts;
//   * a packed operand (weights stored as 16-row x 32-column tiles, see packed_row) keeps its
//     tile order: a 16-row block of one stage is two consecutive tiles, 2 KB contiguous in HBM.
// A problem type P supplies, per operand, a base pointer for the workgroup and, per lane and copy
// instruction, the 32-bit byte offset of the stage-0 source (rows outside the problem are
// clamped to valid rows; their results are never stored), whether each operand is packed
// (which fixes the step per stage), the number of stages and the epilogue.
#pragma once

#include "common.hpp"

namespace lmoe {

template <int BM, int BN, int NS>
struct PipeShape {
    static constexpr int kBM = BM, kBN = BN, kNS = NS;
    static constexpr int kWM = BM / 2, kWN = BN / 2;  // wave tile
    static constexpr int kMB = kWM / 32, kNB = kWN / 32;
    static constexpr int kAI = BM / 8, kBI = BN / 8;      // 1 KB copy instructions per stage
    static constexpr int kAIW = kAI / 4, kBIW = kBI / 4;  // per wave
    static_assert(kAI % 4 == 0 && kBI % 4 == 0, "copies split over 4 waves");
    static constexpr int kLoadsPerStage = kAIW + kBIW;
    static constexpr int kStageUnits = (BM + BN) * 8;  // 16-byte units per stage
    static_assert(NS * kStageUnits * 16 <= 160 * 1024, "LDS budget");
};

// Byte step from one stage to the next: row-major rows advance 64 columns (128 bytes); a
// packed 16-row block advances two 1 KB tiles.
constexpr int kRowMajorStep = 128, kPackedStep = 2048;

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ void lds_copy16(const void* g, uint4* lds_block) {
    __builtin_amdgcn_global_load_lds(g, (lds_ptr_t)lds_block, 16, 0, 0);
}

// Row of copy instruction i for this lane (row-major operands: rows 8i .. 8i+7).
__device__ __forceinline__ int rowmajor_row(int i, int lane) { return 8 * i + (lane >> 3); }

// Byte offset of this lane's 16-byte chunk of copy instruction i at stage 0, for a row-major
// source row that starts `row_bytes` bytes after the operand base.
__device__ __forceinline__ uint32_t rowmajor_off(uint32_t row_bytes, int i, int lane) {
    const int chunk = (lane & 7) ^ (rowmajor_row(i, lane) & 7);
    return row_bytes + chunk * 16;
}

// Byte offset (from the packed matrix base) of copy instruction i: tile (i & 1) of 16-row block nb.
__device__ __forceinline__ uint32_t packed_off(int nb, int i, int K, int lane) {
    return (uint32_t)(((nb * (K / 32) + (i & 1)) * 64 + lane) * 16);
}

// Workgroup barrier without a memory fence: the copies a stage needs are waited for explicitly
// (vmcnt), so the fence that __syncthreads implies would only drain the copies still in flight.
// The empty asm statements keep the compiler from moving LDS accesses across the barrier.
__device__ __forceinline__ void stage_barrier() {
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
}

// s_waitcnt with only vmcnt constrained (expcnt and lgkmcnt at their maxima)
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// waits until at most `left` later stages of this wave's copies are outstanding
template <int LPS, int NS>
__device__ __forceinline__ void wait_stage(int left) {
    if constexpr (NS == 2) {
        wait_vm<0>();  // only the stage being waited for is in flight
        return;
    }
    if constexpr (NS >= 4) {
        if (left >= 2) {
            wait_vm<2 * LPS>();
            return;
        }
    }
    if (left >= 1)
        wait_vm<LPS>();
    else
        wait_vm<0>();
}

// 16-byte unit of (row, 8-column unit u of the stage) in an operand block
template <bool PACKED>
__device__ __forceinline__ int frag_pos(int row, int u) {
    if constexpr (PACKED)
        return ((row >> 4) * 2 + (u >> 2)) * 64 + (u & 3) * 16 + (row & 15);
    else
        return row * 8 + (u ^ (row & 7));
}

// One output tile: the NS-stage copy pipeline over K, then the epilogue.  Every wave of the
// workgroup calls it; the stage buffers must not be in use by any wave.
template <class S, class P>
__device__ __forceinline__ void pipe_tile(const P& p, const typename P::Ctx& ctx, uint4* st0, uint4* st1, uint4* st2,
                                          uint4* st3) {
    constexpr int NS = S::kNS;
    constexpr int LPS = S::kLoadsPerStage;
    static_assert(NS >= 2 && NS <= 4, "two to four stages");

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int nk = p.k_stages(ctx);

    constexpr int kAStep = P::kAPacked ? kPackedStep : kRowMajorStep;
    constexpr int kBStep = P::kBPacked ? kPackedStep : kRowMajorStep;
    // copy sources: a uniform base per operand and per-lane 32-bit byte offsets
    const uint8_t* abase = p.a_base(ctx);
    const uint8_t* bbase = p.b_base(ctx);
    uint32_t as[S::kAIW], bs[S::kBIW];
#pragma unroll
    for (int i = 0; i < S::kAIW; ++i) as[i] = p.src_a(ctx, wave * S::kAIW + i, lane);
#pragma unroll
    for (int i = 0; i < S::kBIW; ++i) bs[i] = p.src_b(ctx, wave * S::kBIW + i, lane);

    // stage buffer: A block (BM rows) then B block (BN rows)
    auto issue = [&](uint4* buf, int kt) {
#pragma unroll
        for (int i = 0; i < S::kAIW; ++i)
            lds_copy16(abase + (as[i] + (uint32_t)(kt * kAStep)), buf + (wave * S::kAIW + i) * 64);
#pragma unroll
        for (int i = 0; i < S::kBIW; ++i)
            lds_copy16(bbase + (bs[i] + (uint32_t)(kt * kBStep)), buf + S::kBM * 8 + (wave * S::kBIW + i) * 64);
    };

    f32x16 acc[S::kMB][S::kNB];
#pragma unroll
    for (int i = 0; i < S::kMB; ++i)
#pragma unroll
        for (int j = 0; j < S::kNB; ++j) acc[i][j] = f32x16{};

    const int fr = lane & 31;
    const int fq = lane >> 5;
    auto compute = [&](const uint4* buf) {
        const uint4* A = buf;
        const uint4* B = buf + S::kBM * 8;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            if constexpr (S::kMB * S::kNB >= 16) __builtin_amdgcn_sched_barrier(0);  // bound live fragments
            const int u = 2 * ks + fq;
            uint4 af[S::kMB], bfv[S::kNB];
#pragma unroll
            for (int i = 0; i < S::kMB; ++i) af[i] = A[frag_pos<P::kAPacked>(wm * S::kWM + i * 32 + fr, u)];
#pragma unroll
            for (int j = 0; j < S::kNB; ++j) bfv[j] = B[frag_pos<P::kBPacked>(wn * S::kWN + j * 32 + fr, u)];
#pragma unroll
            for (int i = 0; i < S::kMB; ++i)
#pragma unroll
                for (int j = 0; j < S::kNB; ++j) acc[i][j] = mfma32(af[i], bfv[j], acc[i][j]);
        }
    };

    // prologue: stages 0 .. NS-2 in flight
    if (nk > 0) issue(st0, 0);
    if constexpr (NS >= 3)
        if (nk > 1) issue(st1, 1);
    if constexpr (NS == 4)
        if (nk > 2) issue(st2, 2);

    // step for stage kt + s: wait for this wave's copies of it, barrier (every wave's copies
    // landed and every wave is done with the previous stage), refill the buffer the previous
    // stage used with stage kt + s + NS - 1, multiply stage kt + s
#define LMOE_PIPE_STEP(S_, CUR_, NEXT_)                              \
    if (kt + S_ < nk) {                                              \
        wait_stage<LPS, NS>(min(nk - 1 - (kt + S_), NS - 2));        \
        stage_barrier();                                             \
        if (kt + S_ + NS - 1 < nk) issue(NEXT_, kt + S_ + NS - 1);   \
        compute(CUR_);                                               \
    }
    if constexpr (NS == 4) {
        for (int kt = 0; kt < nk; kt += 4) {
            LMOE_PIPE_STEP(0, st0, st3)
            LMOE_PIPE_STEP(1, st1, st0)
            LMOE_PIPE_STEP(2, st2, st1)
            LMOE_PIPE_STEP(3, st3, st2)
        }
    } else if constexpr (NS == 3) {
        for (int kt = 0; kt < nk; kt += 3) {
            LMOE_PIPE_STEP(0, st0, st2)
            LMOE_PIPE_STEP(1, st1, st0)
            LMOE_PIPE_STEP(2, st2, st1)
        }
    } else {
        for (int kt = 0; kt < nk; kt += 2) {
            LMOE_PIPE_STEP(0, st0, st1)
            LMOE_PIPE_STEP(1, st1, st0)
        }
    }
#undef LMOE_PIPE_STEP

    p.template epilogue<S::kMB, S::kNB>(ctx, acc, wm * S::kWM, wn * S::kWN, lane);
}

// One tile per workgroup; grid (N tiles, M tiles upper bound), XCD-aware order.
template <class S, class P>
__global__ __launch_bounds__(256) void pipe_gemm_kernel(const P p) {
    __shared__ uint4 st0[S::kStageUnits], st1[S::kStageUnits];
    __shared__ uint4 st2[S::kNS >= 3 ? S::kStageUnits : 1], st3[S::kNS == 4 ? S::kStageUnits : 1];
    typename P::Ctx ctx;
    int m_tile, n_tile;
    xcd_tile(m_tile, n_tile);
    if (!p.tile(m_tile, n_tile, ctx)) return;
    pipe_tile<S, P>(p, ctx, st0, st1, st2, st3);
}

// Persistent form: gridDim.x workgroups (about one per CU) walk the tiles that exist (the M-tile
// count is read on the device).  The tiles are split into g = min(8, gridDim.x) equal contiguous
// ranges, one per XCD (workgroups are handed to the XCDs round-robin), and a group's workgroups
// take the tiles of its range in turn, so the N tiles of one M tile run close together on one
// XCD.  Every tile of every range is taken by some workgroup.
template <class S, class P>
__global__ __launch_bounds__(256) void pipe_gemm_persistent(const P p, int n_tiles) {
    __shared__ uint4 st0[S::kStageUnits], st1[S::kStageUnits];
    __shared__ uint4 st2[S::kNS >= 3 ? S::kStageUnits : 1], st3[S::kNS == 4 ? S::kStageUnits : 1];
    const int total = p.m_tiles() * n_tiles;
    const int g = min(8, (int)gridDim.x);  // groups (XCDs) that have at least one workgroup
    const int x = blockIdx.x % g, wi = blockIdx.x / g;
    const int nwx = ((int)gridDim.x - x + g - 1) / g;  // workgroups in this group
    const int lo = (int)((long)total * x / g), hi = (int)((long)total * (x + 1) / g);
    for (int l = lo + wi; l < hi; l += nwx) {
        typename P::Ctx ctx;
        if (!p.tile(l / n_tiles, l % n_tiles, ctx)) continue;  // uniform over the workgroup
        stage_barrier();  // every wave is done with the previous tile's stage buffers
        pipe_tile<S, P>(p, ctx, st0, st1, st2, st3);
    }
}

}  // namespace lmoe
