// LDS-tiled bf16 MFMA GEMM for batches of many tokens: C[m][n] = sum_k A[m][k] * B[n][k].
//
// Both operands are K-contiguous rows (activations [M][K], weights stored output-major
// [N][K]), which is the operand layout of v_mfma_f32_32x32x16_bf16: every lane reads 16
// contiguous bytes of one row.  One workgroup = 4 waves (256 threads) computes a BM x BN tile
// with BK = 64; global -> register -> LDS staging is double buffered with one barrier per
// k-tile, and LDS rows (128 B) are stored with their 16-B chunks XOR-swizzled by ((row >> 1) & 7)
// so that the 16 consecutive rows a fragment read touches at a time spread over all LDS banks.
//
// A problem type P supplies the tile mapping, row addressing, loads (which may gather rows,
// dequantise or split fp32 into hi/lo bf16 pairs) and the epilogue.
#pragma once

#include "common.hpp"

namespace lmoe {

template <int BM, int BN, int WAVES_M, int WAVES_N>
struct TileShape {
    static constexpr int kBM = BM, kBN = BN, kBK = 64;
    static constexpr int kWavesM = WAVES_M, kWavesN = WAVES_N;
    static constexpr int kWM = BM / WAVES_M, kWN = BN / WAVES_N;
    static constexpr int kMB = kWM / 32, kNB = kWN / 32;
    static_assert(WAVES_M * WAVES_N == 4, "4 waves per workgroup");
    static_assert(kWM % 32 == 0 && kWN % 32 == 0, "wave tile is a multiple of 32x32");
    static constexpr int kAPerThread = BM * 8 / 256;
    static constexpr int kBPerThread = BN * 8 / 256;
    static_assert(kAPerThread >= 1 && kBPerThread >= 1, "tile too small");
};

__device__ __forceinline__ int swz(int row, int chunk) { return row * 8 + (chunk ^ ((row >> 1) & 7)); }

template <class S, class P>
__global__ __launch_bounds__(256) void tile_gemm_kernel(const P p) {
    __shared__ uint4 sA[2][S::kBM * 8];
    __shared__ uint4 sB[2][S::kBN * 8];

    typename P::Ctx ctx;
    int m_tile, n_tile;
    xcd_tile(m_tile, n_tile);  // grid: (N tiles, M tiles)
    if (!p.tile(m_tile, n_tile, ctx)) return;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / S::kWavesN;
    const int wn = wave % S::kWavesN;
    const int lc = tid & 7;   // 16-B chunk this thread stages
    const int lr = tid >> 3;  // first row this thread stages (then +32, +64, ...)

    typename P::RowA arow[S::kAPerThread];
    typename P::RowB brow[S::kBPerThread];
#pragma unroll
    for (int i = 0; i < S::kAPerThread; ++i) arow[i] = p.row_a(ctx, lr + 32 * i);
#pragma unroll
    for (int i = 0; i < S::kBPerThread; ++i) brow[i] = p.row_b(ctx, lr + 32 * i);

    const int nk = p.k_tiles(ctx);
    uint4 ra[S::kAPerThread], rb[S::kBPerThread];
#pragma unroll
    for (int i = 0; i < S::kAPerThread; ++i) ra[i] = p.load_a(ctx, arow[i], 0, lc);
#pragma unroll
    for (int i = 0; i < S::kBPerThread; ++i) rb[i] = p.load_b(ctx, brow[i], 0, lc);
#pragma unroll
    for (int i = 0; i < S::kAPerThread; ++i) sA[0][swz(lr + 32 * i, lc)] = ra[i];
#pragma unroll
    for (int i = 0; i < S::kBPerThread; ++i) sB[0][swz(lr + 32 * i, lc)] = rb[i];
    __syncthreads();

    f32x16 acc[S::kMB][S::kNB];
#pragma unroll
    for (int i = 0; i < S::kMB; ++i)
#pragma unroll
        for (int j = 0; j < S::kNB; ++j) acc[i][j] = f32x16{};

    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < nk;
        if (more) {
#pragma unroll
            for (int i = 0; i < S::kAPerThread; ++i) ra[i] = p.load_a(ctx, arow[i], kt + 1, lc);
#pragma unroll
            for (int i = 0; i < S::kBPerThread; ++i) rb[i] = p.load_b(ctx, brow[i], kt + 1, lc);
        }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int chunk = ks * 2 + (lane >> 5);
            uint4 af[S::kMB], bfv[S::kNB];
#pragma unroll
            for (int i = 0; i < S::kMB; ++i) af[i] = sA[cur][swz(wm * S::kWM + i * 32 + (lane & 31), chunk)];
#pragma unroll
            for (int j = 0; j < S::kNB; ++j) bfv[j] = sB[cur][swz(wn * S::kWN + j * 32 + (lane & 31), chunk)];
#pragma unroll
            for (int i = 0; i < S::kMB; ++i)
#pragma unroll
                for (int j = 0; j < S::kNB; ++j) acc[i][j] = mfma32(af[i], bfv[j], acc[i][j]);
        }
        if (more) {
#pragma unroll
            for (int i = 0; i < S::kAPerThread; ++i) sA[cur ^ 1][swz(lr + 32 * i, lc)] = ra[i];
#pragma unroll
            for (int i = 0; i < S::kBPerThread; ++i) sB[cur ^ 1][swz(lr + 32 * i, lc)] = rb[i];
        }
        __syncthreads();
    }

    p.template epilogue<S::kMB, S::kNB>(ctx, acc, wm * S::kWM, wn * S::kWN, lane);
}

// Row/column of register r of lane `lane` inside a 32x32 MFMA block.
__device__ __forceinline__ int frag32_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }
__device__ __forceinline__ int frag32_col(int lane) { return lane & 31; }

}  // namespace lmoe
