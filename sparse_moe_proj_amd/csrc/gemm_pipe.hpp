// Pipelined bf16 MFMA GEMM for batches of many tokens: C[m][n] = sum_k A[m][k] * B[n][k].
//
// One workgroup of WR x WC waves computes a BM x BN tile (each wave (BM/WR) x (BN/WC) with
// v_mfma_f32_32x32x16_bf16).  K advances in stages of 64 columns.  Each stage's operands are
// copied straight from global memory into LDS with global_load_lds_dwordx4 (no register
// staging), NS stages deep, so the copies of the next NS-1 stages are in flight while one
// stage is multiplied; one barrier per stage.
//
// A copy instruction moves 1 KB: lane l writes LDS position l of the instruction's block, and
// the lane picks its global source so that
//   * a row-major operand block holds 8 rows x 128 bytes (a full cache line per row), with the
//     16-byte chunks of row r stored XOR-swizzled by ((r >> 1) & 7): a fragment read takes one
//     chunk from each of 16 consecutive rows, and a row's 32 banks are set by its parity and the
//     chunk, so the 8 rows of each parity must use 8 different chunks (swizzling by (r & 7) gave
//     rows r and r + 8 the same banks);
//   * a packed operand (weights stored as 16-row x 32-column tiles, see packed_row) keeps its
//     tile order: a 16-row block of one stage is two consecutive tiles, 2 KB contiguous in HBM.
// A problem type P supplies, per operand, a base pointer for the workgroup and, per lane and copy
// instruction, the 32-bit byte offset of the stage-0 source (rows outside the problem are
// clamped to valid rows; their results are never stored), whether each operand is packed
// (which fixes the step per stage), the number of stages and the epilogue.
#pragma once

#include "common.hpp"

namespace lmoe {

template <int BM, int BN, int NS, int WR = 2, int WC = 2>
struct PipeShape {
    static constexpr int kBM = BM, kBN = BN, kNS = NS;
    static constexpr int kWR = WR, kWC = WC, kWaves = WR * WC, kThreads = 64 * WR * WC;
    static constexpr int kWM = BM / WR, kWN = BN / WC;  // wave tile
    static constexpr int kMB = kWM / 32, kNB = kWN / 32;
    static constexpr int kAI = BM / 8, kBI = BN / 8;                // 1 KB copy instructions per stage
    static constexpr int kAIW = kAI / kWaves, kBIW = kBI / kWaves;  // per wave
    static_assert(kAI % kWaves == 0 && kBI % kWaves == 0, "copies split over the waves");
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
    const int chunk = (lane & 7) ^ ((rowmajor_row(i, lane) >> 1) & 7);
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
        return row * 8 + (u ^ ((row >> 1) & 7));
}

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const uint4* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint4*)p;
}

// Fragment reads of one k step: MB + NB ds_read_b128 in one block that also waits for them.
// The copies into other stage buffers are still in flight at this point; keeping these reads out
// of the compiler's view stops it from waiting for those copies (it cannot tell the buffers
// apart across the K loop's back edge).  Outputs are early-clobber, so no register of an address
// still to be used receives data, and the block returns only once every read has landed.
template <int MB, int NB>
__device__ __forceinline__ void lds_read_frags(const uint32_t (&aa)[MB], const uint32_t (&ba)[NB], uint4 (&af)[MB],
                                               uint4 (&bf)[NB]) {
    if constexpr (MB == 2 && NB == 4) {
        __asm__ volatile(
            "ds_read_b128 %0, %6\n\t"
            "ds_read_b128 %1, %7\n\t"
            "ds_read_b128 %2, %8\n\t"
            "ds_read_b128 %3, %9\n\t"
            "ds_read_b128 %4, %10\n\t"
            "ds_read_b128 %5, %11\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(af[0]), "=&v"(af[1]), "=&v"(bf[0]), "=&v"(bf[1]), "=&v"(bf[2]), "=&v"(bf[3])
            : "v"(aa[0]), "v"(aa[1]), "v"(ba[0]), "v"(ba[1]), "v"(ba[2]), "v"(ba[3]));
    } else if constexpr (MB == 4 && NB == 2) {
        __asm__ volatile(
            "ds_read_b128 %0, %6\n\t"
            "ds_read_b128 %1, %7\n\t"
            "ds_read_b128 %2, %8\n\t"
            "ds_read_b128 %3, %9\n\t"
            "ds_read_b128 %4, %10\n\t"
            "ds_read_b128 %5, %11\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(af[0]), "=&v"(af[1]), "=&v"(af[2]), "=&v"(af[3]), "=&v"(bf[0]), "=&v"(bf[1])
            : "v"(aa[0]), "v"(aa[1]), "v"(aa[2]), "v"(aa[3]), "v"(ba[0]), "v"(ba[1]));
    } else if constexpr (MB == 2 && NB == 2) {
        __asm__ volatile(
            "ds_read_b128 %0, %4\n\t"
            "ds_read_b128 %1, %5\n\t"
            "ds_read_b128 %2, %6\n\t"
            "ds_read_b128 %3, %7\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(af[0]), "=&v"(af[1]), "=&v"(bf[0]), "=&v"(bf[1])
            : "v"(aa[0]), "v"(aa[1]), "v"(ba[0]), "v"(ba[1]));
    } else {
        static_assert(MB == 4 && NB == 4, "wave tiles of 64 or 128 rows and columns");
        __asm__ volatile(
            "ds_read_b128 %0, %8\n\t"
            "ds_read_b128 %1, %9\n\t"
            "ds_read_b128 %2, %10\n\t"
            "ds_read_b128 %3, %11\n\t"
            "ds_read_b128 %4, %12\n\t"
            "ds_read_b128 %5, %13\n\t"
            "ds_read_b128 %6, %14\n\t"
            "ds_read_b128 %7, %15\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(af[0]), "=&v"(af[1]), "=&v"(af[2]), "=&v"(af[3]), "=&v"(bf[0]), "=&v"(bf[1]), "=&v"(bf[2]),
              "=&v"(bf[3])
            : "v"(aa[0]), "v"(aa[1]), "v"(aa[2]), "v"(aa[3]), "v"(ba[0]), "v"(ba[1]), "v"(ba[2]), "v"(ba[3]));
    }
}

// Copy sources of one tile for this lane: a uniform base per operand and per-lane 32-bit byte
// offsets of the stage-0 source of each copy instruction this wave issues.
template <class S>
struct PipeCopies {
    const uint8_t* abase;
    const uint8_t* bbase;
    uint32_t as[S::kAIW], bs[S::kBIW];
};

template <class S, class P>
__device__ __forceinline__ PipeCopies<S> pipe_copies(const P& p, const typename P::Ctx& ctx, int wave, int lane) {
    PipeCopies<S> c;
    c.abase = p.a_base(ctx);
    c.bbase = p.b_base(ctx);
#pragma unroll
    for (int i = 0; i < S::kAIW; ++i) c.as[i] = p.src_a(ctx, wave * S::kAIW + i, lane);
#pragma unroll
    for (int i = 0; i < S::kBIW; ++i) c.bs[i] = p.src_b(ctx, wave * S::kBIW + i, lane);
    return c;
}

// Stage kt of the tile into stage buffer buf (A block of BM rows, then B block of BN rows).
template <class S, class P>
__device__ __forceinline__ void pipe_issue(const PipeCopies<S>& c, uint4* buf, int kt, int wave) {
    constexpr int kAStep = P::kAPacked ? kPackedStep : kRowMajorStep;
    constexpr int kBStep = P::kBPacked ? kPackedStep : kRowMajorStep;
#pragma unroll
    for (int i = 0; i < S::kAIW; ++i)
        lds_copy16(c.abase + (c.as[i] + (uint32_t)(kt * kAStep)), buf + (wave * S::kAIW + i) * 64);
#pragma unroll
    for (int i = 0; i < S::kBIW; ++i)
        lds_copy16(c.bbase + (c.bs[i] + (uint32_t)(kt * kBStep)), buf + S::kBM * 8 + (wave * S::kBIW + i) * 64);
}

// Stages 0 .. NS-2 of a tile with nk stages into the first stage buffers.
template <class S, class P>
__device__ __forceinline__ void pipe_prologue(const PipeCopies<S>& c, int nk, uint4* st0, uint4* st1, uint4* st2,
                                              int wave) {
    if (nk > 0) pipe_issue<S, P>(c, st0, 0, wave);
    if constexpr (S::kNS >= 3)
        if (nk > 1) pipe_issue<S, P>(c, st1, 1, wave);
    if constexpr (S::kNS == 4)
        if (nk > 2) pipe_issue<S, P>(c, st2, 2, wave);
}

// The K loop of one tile whose prologue stages are in flight: for stage kt + s, wait for this
// wave's copies of it, barrier (every wave's copies landed and every wave is done with the
// previous stage), refill the buffer the previous stage used with stage kt + s + NS - 1,
// multiply stage kt + s.  Accumulates into acc (zeroed here).
template <class S, class P>
__device__ __forceinline__ void pipe_k_loop(const PipeCopies<S>& c, int nk, f32x16 (&acc)[S::kMB][S::kNB],
                                            uint4* st0, uint4* st1, uint4* st2, uint4* st3, int wave, int lane) {
    constexpr int NS = S::kNS;
    constexpr int LPS = S::kLoadsPerStage;
    static_assert(NS >= 2 && NS <= 4, "two to four stages");
    const int wm = wave / S::kWC, wn = wave % S::kWC;
#pragma unroll
    for (int i = 0; i < S::kMB; ++i)
#pragma unroll
        for (int j = 0; j < S::kNB; ++j) acc[i][j] = f32x16{};

    const int fr = lane & 31;
    const int fq = lane >> 5;
    auto compute = [&](const uint4* buf) {
        const uint32_t A = lds_addr(buf);
        const uint32_t B = A + S::kBM * 8 * 16;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int u = 2 * ks + fq;
            uint32_t aa[S::kMB], ba[S::kNB];
#pragma unroll
            for (int i = 0; i < S::kMB; ++i) aa[i] = A + 16 * frag_pos<P::kAPacked>(wm * S::kWM + i * 32 + fr, u);
#pragma unroll
            for (int j = 0; j < S::kNB; ++j) ba[j] = B + 16 * frag_pos<P::kBPacked>(wn * S::kWN + j * 32 + fr, u);
            uint4 af[S::kMB], bfv[S::kNB];
            lds_read_frags<S::kMB, S::kNB>(aa, ba, af, bfv);
#pragma unroll
            for (int i = 0; i < S::kMB; ++i)
#pragma unroll
                for (int j = 0; j < S::kNB; ++j) acc[i][j] = mfma32(af[i], bfv[j], acc[i][j]);
        }
    };

#define LMOE_PIPE_STEP(S_, CUR_, NEXT_)                                             \
    if (kt + S_ < nk) {                                                             \
        wait_stage<LPS, NS>(min(nk - 1 - (kt + S_), NS - 2));                       \
        stage_barrier();                                                            \
        if (kt + S_ + NS - 1 < nk) pipe_issue<S, P>(c, NEXT_, kt + S_ + NS - 1, wave); \
        compute(CUR_);                                                              \
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
}

// One tile per workgroup; grid (N tiles, M tiles upper bound), XCD-aware order.
template <class S, class P>
__global__ __launch_bounds__(S::kThreads) void pipe_gemm_kernel(const P p) {
    __shared__ uint4 st0[S::kStageUnits], st1[S::kStageUnits];
    __shared__ uint4 st2[S::kNS >= 3 ? S::kStageUnits : 1], st3[S::kNS == 4 ? S::kStageUnits : 1];
    typename P::Ctx ctx;
    int m_tile, n_tile;
    xcd_tile(m_tile, n_tile);
    if (!p.tile(m_tile, n_tile, ctx)) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rb = (wave / S::kWC) * S::kWM, cb = (wave % S::kWC) * S::kWN;
    const int nk = p.k_stages(ctx);
    const PipeCopies<S> c = pipe_copies<S>(p, ctx, wave, lane);
    pipe_prologue<S, P>(c, nk, st0, st1, st2, wave);
    f32x16 acc[S::kMB][S::kNB];
    pipe_k_loop<S, P>(c, nk, acc, st0, st1, st2, st3, wave, lane);
    const auto prep = p.template prep<S::kMB>(ctx, rb, lane);
    p.template store<S::kMB, S::kNB>(ctx, acc, prep, rb, cb, lane);
}

// Persistent form: gridDim.x workgroups (about one per CU) walk the tiles that exist (the M-tile
// count is read on the device).  The tiles are split into g = min(8, gridDim.x) equal contiguous
// ranges, one per XCD (workgroups are handed to the XCDs round-robin), and a group's workgroups
// take the tiles of its range in turn, so the N tiles of one M tile run close together on one
// XCD.  Every tile of every range is taken by some workgroup.
//
// Tiles overlap: once a tile's K loop is done, the workgroup reads what the epilogue needs
// (P::prep) and the next tile's copy sources, issues the next tile's first stages, and only then
// stores the finished tile, so the stores and the next tile's first copies are in flight
// together.  No global load is issued after the prefetch until the next K loop (a wait for such
// a load would also wait for the prefetch).
template <class S, class P>
__global__ __launch_bounds__(S::kThreads) void pipe_gemm_persistent(const P p, int n_tiles) {
    __shared__ uint4 st0[S::kStageUnits], st1[S::kStageUnits];
    __shared__ uint4 st2[S::kNS >= 3 ? S::kStageUnits : 1], st3[S::kNS == 4 ? S::kStageUnits : 1];
    const int total = p.m_tiles() * n_tiles;
    const int g = min(8, (int)gridDim.x);  // groups (XCDs) that have at least one workgroup
    const int x = blockIdx.x % g, wi = blockIdx.x / g;
    const int nwx = ((int)gridDim.x - x + g - 1) / g;  // workgroups in this group
    const int lo = (int)((long)total * x / g), hi = (int)((long)total * (x + 1) / g);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rb = (wave / S::kWC) * S::kWM, cb = (wave % S::kWC) * S::kWN;

    // the next valid tile at or after l (uniform over the workgroup); false when none is left
    auto next_tile = [&](int& l, typename P::Ctx& ctx) {
        for (; l < hi; l += nwx)
            if (p.tile(l / n_tiles, l % n_tiles, ctx)) return true;
        return false;
    };
    int l = lo + wi;
    typename P::Ctx ctx;
    if (!next_tile(l, ctx)) return;
    int nk = p.k_stages(ctx);
    PipeCopies<S> c = pipe_copies<S>(p, ctx, wave, lane);
    pipe_prologue<S, P>(c, nk, st0, st1, st2, wave);
    f32x16 acc[S::kMB][S::kNB];
    while (true) {
        pipe_k_loop<S, P>(c, nk, acc, st0, st1, st2, st3, wave, lane);
        const auto prep = p.template prep<S::kMB>(ctx, rb, lane);
        int ln = l + nwx;
        typename P::Ctx nctx;
        const bool more = next_tile(ln, nctx);
        int nnk = 0;
        PipeCopies<S> nc;
        if (more) {
            nnk = p.k_stages(nctx);
            nc = pipe_copies<S>(p, nctx, wave, lane);
        }
        stage_barrier();  // every wave is done with this tile's stage buffers
        if (more) pipe_prologue<S, P>(nc, nnk, st0, st1, st2, wave);
        p.template store<S::kMB, S::kNB>(ctx, acc, prep, rb, cb, lane);
        if (!more) break;
        l = ln;
        ctx = nctx;
        nk = nnk;
        c = nc;
    }
}

}  // namespace lmoe
