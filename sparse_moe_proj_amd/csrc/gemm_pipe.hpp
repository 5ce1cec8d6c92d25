// Pipelined bf16 MFMA GEMM for batches of many tokens: C[m][n] = sum_k A[m][k] * B[n][k].
//
// One workgroup of WR x WC waves computes a BM x BN tile (each wave (BM/WR) x (BN/WC) with
// v_mfma_f32_32x32x16_bf16).  K advances in stages of BK columns (64, or 32 for a deeper
// pipeline in the same LDS).  Each stage's operands are copied straight from global memory into
// LDS with global_load_lds_dwordx4 (no register staging), NS stages deep, so the copies of the
// next NS-1 stages are in flight while one stage is multiplied; one barrier per stage.
//
// A copy instruction moves 1 KB: lane l writes LDS position l of the instruction's block, and
// the lane picks its global source so that
//   * a row-major operand block holds 512/BK rows x 2 BK bytes (BK = 64: a full cache line per
//     row), with the U = BK/8 16-byte chunks of row r stored XOR-swizzled by (r U / 16) mod U: a
//     fragment read takes one chunk from each of 16 consecutive rows, the 64 banks of 4 bytes
//     hold 16/U rows side by side, so the U rows of those 16 that share banks must use U
//     different chunks (for BK = 64 the swizzle (r >> 1) & 7; swizzling by (r & 7) gave rows r
//     and r + 8 the same banks);
//   * a packed operand (weights stored as 16-row x 32-column tiles, see packed_row) keeps its
//     tile order: a 16-row block of one stage is BK/32 consecutive 1 KB tiles, contiguous in HBM.
// A problem type P supplies, per operand, a base pointer for the workgroup and, per lane and copy
// instruction, the 32-bit byte offset of the stage-0 source (rows outside the problem are
// clamped to valid rows; their results are never stored), whether each operand is packed
// (which fixes the step per stage), the number of stages and the epilogue.  The MFMAs take the B
// fragment as their first operand, so each 32 x 32 accumulator block holds the transposed
// product: register r of lane l is row l % 32 and column 8 (r / 4) + 4 (l / 32) + r % 4 of the
// block, four consecutive columns of one row per group of four registers, which the epilogues
// store 8 or 16 bytes at a time.
#pragma once

#include "common.hpp"

namespace lmoe {

template <int BM, int BN, int NS, int WR = 2, int WC = 2, int BK = 64>
struct PipeShape {
    static constexpr int kBM = BM, kBN = BN, kNS = NS, kBK = BK;
    static constexpr int kU = BK / 8;  // 16-byte units of a row per stage
    static_assert(BK == 64 || BK == 32, "stages of 64 or 32 columns");
    static constexpr int kWR = WR, kWC = WC, kWaves = WR * WC, kThreads = 64 * WR * WC;
    static constexpr int kWM = BM / WR, kWN = BN / WC;  // wave tile
    static constexpr int kMB = kWM / 32, kNB = kWN / 32;
    static constexpr int kAI = BM * kU / 64, kBI = BN * kU / 64;    // 1 KB copy instructions per stage
    static constexpr int kAIW = kAI / kWaves, kBIW = kBI / kWaves;  // per wave
    static_assert(kAI % kWaves == 0 && kBI % kWaves == 0, "copies split over the waves");
    static constexpr int kLoadsPerStage = kAIW + kBIW;
    static constexpr int kStageUnits = (BM + BN) * kU;  // 16-byte units per stage
    static_assert(NS * kStageUnits * 16 <= 160 * 1024, "LDS budget");
    // byte step from one stage to the next: a row-major row advances BK columns, a packed 16-row
    // block BK/32 tiles of 1 KB
    static constexpr int kRowMajorStep = 2 * BK, kPackedStep = 32 * BK;
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ void lds_copy16(const void* g, uint4* lds_block) {
    __builtin_amdgcn_global_load_lds(g, (lds_ptr_t)lds_block, 16, 0, 0);
}

// Swizzle of row r's 16-byte chunks in a row-major stage block of U chunks per row.
template <int U = 8>
__device__ __forceinline__ int rowmajor_swz(int r) { return (r * U / 16) & (U - 1); }

// Row of copy instruction i for this lane (row-major operands: rows (64/U) i .. (64/U) i + 64/U - 1).
template <int U = 8>
__device__ __forceinline__ int rowmajor_row(int i, int lane) { return (64 / U) * i + lane / U; }

// Byte offset of this lane's 16-byte chunk of copy instruction i at stage 0, for a row-major
// source row that starts `row_bytes` bytes after the operand base.
template <int U = 8>
__device__ __forceinline__ uint32_t rowmajor_off(uint32_t row_bytes, int i, int lane) {
    const int chunk = (lane & (U - 1)) ^ rowmajor_swz<U>(rowmajor_row<U>(i, lane));
    return row_bytes + chunk * 16;
}

// Byte offset (from the packed matrix base) of copy instruction i: tile i mod (U/4) of 16-row
// block nb (the stage's U/4 tiles of that block).
template <int U = 8>
__device__ __forceinline__ uint32_t packed_off(int nb, int i, int K, int lane) {
    return (uint32_t)(((nb * (K / 32) + i % (U / 4)) * 64 + lane) * 16);
}

// First 16-row block of packed copy instruction i
template <int U = 8>
__device__ __forceinline__ int packed_block(int i) { return i / (U / 4); }

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

// 16-byte unit of (row, 8-column unit u of the stage) in an operand block of U units per row
template <bool PACKED, int U = 8>
__device__ __forceinline__ int frag_pos(int row, int u) {
    if constexpr (PACKED)
        return ((row >> 4) * (U / 4) + (u >> 2)) * 64 + (u & 3) * 16 + (row & 15);
    else
        return row * U + (u ^ rowmajor_swz<U>(row));
}

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const uint4* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint4*)p;
}

// LDS writes and reads of a tile's staged output (outside the K loop).  The reads run while the
// next tile's first copies fill another stage buffer; in asm, with their wait in the same block
// (early-clobber outputs, so no address register still in use receives data), they keep the
// compiler from waiting for those copies as well.
__device__ __forceinline__ void lds_write_b64(uint32_t addr, uint2 v) {
    __asm__ volatile("ds_write_b64 %0, %1" ::"v"(addr), "v"(v) : "memory");
}
__device__ __forceinline__ void lds_wait() { __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void lds_read8_b128(const uint32_t (&a)[8], uint4 (&v)[8]) {
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
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
        : "memory");
}

// A tile of bf16 outputs stored through the stage buffers, so that every store instruction
// writes whole row segments (the transposed accumulators give each lane 8 bytes of one row).
// Half h of the tile (the BM/2 rows of the waves with wm = h; WR = 2) goes into stage buffer h
// (buffer 2 for the second half when a tile's prologue also fills buffer 1) as rows of C chunks
// of 16 bytes, chunk c of row r at position c ^ (r % C): the writes (8 bytes of one row per
// lane) and the reads (whole rows) spread over the banks.
//   put(i, j, r4) -> uint2: the 4 bf16 of accumulator group r4 of block (i, j) of this lane,
//       staged in chunk chunk_of(j, r4) of its row (blocks j < NJ are written);
//   row_of(r) -> the output row of tile row r, or -1 for none (read after the first barrier);
//   out + row * stride + col0 + 8 c receives chunk c of a row whose col0 + 8 c < ncols.
// Thread t then reads and stores chunk t % C of rows t / C + (512 / C) k of each half.  With
// RELEASE, issue_next() runs once every wave has read the first half back (the next tile's first
// stages then fill buffer 0 while the second half is stored).
template <class SS, int C, int NJ, bool RELEASE, int MB, int NB, class Put, class ChunkOf, class RowOf, class F>
__device__ __forceinline__ void staged_store_bf16(int lane, int wave, uint4* st0, uint4* st1, uint4* st2, Put&& put,
                                                  ChunkOf&& chunk_of, RowOf&& row_of, uint16_t* out, size_t stride,
                                                  int col0, int ncols, F&& issue_next) {
    static_assert(SS::kWR == 2 && SS::kThreads == 512 && (C == 16 || C == 32), "two wave rows, 16 or 32 chunks");
    constexpr int kRows = SS::kBM / 2;             // rows of a half
    constexpr int kRowBytes = 16 * C;
    static_assert(kRows * kRowBytes <= SS::kStageUnits * 16, "half a tile fits a stage buffer");
    constexpr int kStep = 512 / C;                 // rows read per pass of the workgroup
    constexpr int kPer = kRows / kStep;            // chunks per thread and half
    static_assert(kPer >= 1 && kPer <= 8, "1 to 8 chunks per thread and half");
    const int wm = wave / SS::kWC;
    const uint32_t hbase[2] = {lds_addr(st0), lds_addr(SS::kNS >= 3 ? st2 : st1)};
    lane = opaque(lane);  // the per-lane addresses below are recomputed per tile, not kept across tiles
    {
        const uint32_t base = hbase[wm];
        const int h8 = 8 * (lane >> 5);
        static_for<MB>([&](auto i) {
            const int rl = i * 32 + (lane & 31);
            static_for<NJ>([&](auto j) {
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4)
                    lds_write_b64(base + rl * kRowBytes + ((chunk_of(j, r4) ^ (rl & (C - 1))) * 16) + h8, put(i, j, r4));
            });
        });
    }
    lds_wait();
    stage_barrier();
    const int t = opaque(threadIdx.x), ch = t % C, r0 = t / C;
    int row[2][kPer];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int k = 0; k < kPer; ++k) row[h][k] = row_of(h * kRows + r0 + kStep * k);
    const int col = col0 + 8 * ch;
    auto half = [&](int h, auto&& after_read) {
        uint32_t a[8];
        uint4 v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int r = r0 + kStep * (k < kPer ? k : 0);
            a[k] = hbase[h] + r * kRowBytes + ((ch ^ (r & (C - 1))) * 16);
        }
        lds_read8_b128(a, v);
        after_read();
#pragma unroll
        for (int k = 0; k < kPer; ++k)
            if (row[h][k] >= 0 && col < ncols) *reinterpret_cast<uint4*>(out + (size_t)row[h][k] * stride + col) = v[k];
    };
    half(0, [&] {
        if constexpr (RELEASE) {
            stage_barrier();  // every wave has read the first half back
            issue_next();
        }
    });
    half(1, [] {});
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
    constexpr int kAStep = P::kAPacked ? S::kPackedStep : S::kRowMajorStep;
    constexpr int kBStep = P::kBPacked ? S::kPackedStep : S::kRowMajorStep;
#pragma unroll
    for (int i = 0; i < S::kAIW; ++i)
        lds_copy16(c.abase + (c.as[i] + (uint32_t)(kt * kAStep)), buf + (wave * S::kAIW + i) * 64);
#pragma unroll
    for (int i = 0; i < S::kBIW; ++i)
        lds_copy16(c.bbase + (c.bs[i] + (uint32_t)(kt * kBStep)), buf + S::kBM * S::kU + (wave * S::kBIW + i) * 64);
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
// multiply stage kt + s.  Accumulates into acc (zeroed here).  mrows: the tile's rows that hold
// data (the others only pad it): a wave multiplies only its 32-row blocks that reach into them,
// and a wave with none reads no fragments (it still takes part in the copies and barriers).
template <class S, class P>
__device__ __forceinline__ void pipe_k_loop(const PipeCopies<S>& c, int nk, f32x16 (&acc)[S::kMB][S::kNB],
                                            uint4* st0, uint4* st1, uint4* st2, uint4* st3, int wave, int lane,
                                            int mrows) {
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
    const int nvb = min(S::kMB, max(0, (mrows - wm * S::kWM + 31) / 32));  // 32-row blocks with data
    // A tile whose every 32-row block holds data (all but a segment's last tile) multiplies with
    // plain LDS loads, which the compiler waits for exactly (lgkmcnt): the first k step's
    // fragments are requested right after the barrier, ahead of the next stage's copies, and
    // each k step's MFMAs are interleaved with the loads of the next k step's fragments.
    auto frag_a = [&](int i, int ks) { return frag_pos<P::kAPacked, S::kU>(wm * S::kWM + i * 32 + fr, 2 * ks + fq); };
    auto frag_b = [&](int j, int ks) {
        return S::kBM * S::kU + frag_pos<P::kBPacked, S::kU>(wn * S::kWN + j * 32 + fr, 2 * ks + fq);
    };
    constexpr int NKS = S::kBK / 16;
    // One stage for a wave whose first NV 32-row blocks hold data (NV = kMB but in a segment's
    // last tile), without branches: the A fragments of the other blocks are neither read nor
    // multiplied, and a wave with NV = 0 only issues its share of the copies.
    auto step = [&](auto nvc, const uint4* buf, uint4* nbuf, int nkt) {
        constexpr int NV = decltype(nvc)::value;
        // fa[i] is reloaded with the next k step's fragment as soon as its MFMAs are issued; the
        // B fragments, which every MFMA of a k step reads, alternate between two sets
        uint4 fa[S::kMB], fb[2][S::kNB];
        if constexpr (NV > 0) {
#pragma unroll
            for (int i = 0; i < NV; ++i) fa[i] = buf[frag_a(i, 0)];
#pragma unroll
            for (int j = 0; j < S::kNB; ++j) fb[0][j] = buf[frag_b(j, 0)];
        }
        if (nkt >= 0) pipe_issue<S, P>(c, nbuf, nkt, wave);
        if constexpr (NV > 0) {
            static_for<NKS>([&](auto ksc) {
                constexpr int ks = decltype(ksc)::value, cur = ks & 1, nxt = cur ^ 1;
                constexpr bool more = ks + 1 < NKS;
                if constexpr (more)
#pragma unroll
                    for (int j = 0; j < S::kNB; ++j) fb[nxt][j] = buf[frag_b(j, ks + 1)];
#pragma unroll
                for (int i = 0; i < NV; ++i) {
#pragma unroll
                    for (int j = 0; j < S::kNB; ++j) acc[i][j] = mfma32(fb[cur][j], fa[i], acc[i][j]);
                    if constexpr (more) fa[i] = buf[frag_a(i, ks + 1)];
                }
            });
            // order of the region after the copies, per k step: the next B fragments, then each
            // row block's MFMAs followed by the load of its next A fragment
            static_for<NKS>([&](auto ksc) {
                constexpr bool more = decltype(ksc)::value + 1 < NKS;
                if constexpr (more) __builtin_amdgcn_sched_group_barrier(0x100, S::kNB, 0);  // DS read
                static_for<NV>([&](auto) {
                    __builtin_amdgcn_sched_group_barrier(0x008, S::kNB, 0);  // MFMA
                    if constexpr (more) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                });
            });
        }
    };

#define LMOE_PIPE_STEP(S_, CUR_, NEXT_)                                             \
    if (kt + S_ < nk) {                                                             \
        wait_stage<LPS, NS>(min(nk - 1 - (kt + S_), NS - 2));                       \
        stage_barrier();                                                            \
        const int nkt = kt + S_ + NS - 1 < nk ? kt + S_ + NS - 1 : -1;              \
        step(nvc, CUR_, NEXT_, nkt);                                                \
    }
    // the number of data blocks is fixed for the tile: one compact K loop per value
    auto run = [&](auto nvc) {
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
    };
    static_for<S::kMB + 1>([&](auto nvc) {
        if (nvb == decltype(nvc)::value) run(nvc);
    });
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
    pipe_k_loop<S, P>(c, nk, acc, st0, st1, st2, st3, wave, lane, p.valid_rows(ctx));
    const auto prep = p.template prep<S::kMB>(ctx, rb, lane);
    __syncthreads();  // a problem's prep may stage rows in LDS for the store
    if constexpr (P::kLdsStore)
        p.template store_lds<S>(ctx, acc, prep, rb, cb, lane, wave, st0, st1, st2, [] {});
    else
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
        pipe_k_loop<S, P>(c, nk, acc, st0, st1, st2, st3, wave, lane, p.valid_rows(ctx));
        const auto prep = p.template prep<S::kMB>(ctx, rb, lane);
        int ln = l + nwx;
        typename P::Ctx nctx;
        const bool more = next_tile(ln, nctx);
        int nnk = 0;
        PipeCopies<S> nc;
        if (more) {
            nnk = p.k_stages(nctx);
            nc = pipe_copies<S>(p, nctx, wave, opaque(lane));  // per-lane terms recomputed per tile
        }
        stage_barrier();  // every wave is done with this tile's stage buffers
        if constexpr (P::kLdsStore) {
            // the store stages the tile in the stage buffers and issues the next tile's first
            // stages as soon as the buffers they fill have been read back
            p.template store_lds<S>(ctx, acc, prep, rb, cb, lane, wave, st0, st1, st2, [&] {
                if (more) pipe_prologue<S, P>(nc, nnk, st0, st1, st2, wave);
            });
        } else {
            if (more) pipe_prologue<S, P>(nc, nnk, st0, st1, st2, wave);
            p.template store<S::kMB, S::kNB>(ctx, acc, prep, rb, cb, lane);
        }
        if (!more) break;
        l = ln;
        ctx = nctx;
        nk = nnk;
        c = nc;
    }
}

}  // namespace lmoe
