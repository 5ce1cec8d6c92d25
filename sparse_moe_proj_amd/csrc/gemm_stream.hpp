// Weight-streaming bf16 MFMA kernel for small token batches (decode / speculative verify):
// C[n][t] = sum_k W[n][k] * X[t][k] for 16 weight rows n per workgroup and up to 16 tokens t.
//
// At a handful of tokens the work is bound by reading the weights once from HBM, so the
// weights are the MFMA A operand loaded straight from global memory into registers (16
// contiguous bytes per lane, the v_mfma_f32_16x16x32_bf16 operand layout), and the tokens
// are the B operand (columns >= the batch are zero).  The K dimension is split into KS
// contiguous slices, one per wave, so a workgroup keeps KS x 16 rows' worth of loads in
// flight; the KS partial 16x16 tiles are summed in LDS in wave order (deterministic).
//
// NMAT weight matrices can be streamed against the same tokens (2 for the fused SwiGLU
// gate/up projection).  A problem type P supplies addressing, loads and the epilogue.
#pragma once

#include "common.hpp"

namespace lmoe {

template <int KS, int NMAT, class P>
__global__ __launch_bounds__(64 * KS) void stream_gemm_kernel(const P p) {
    __shared__ float red[KS][NMAT][256];

    typename P::Ctx ctx;
    if (!p.tile(blockIdx.x, ctx)) return;  // grid.x: token tile / work-list entry
    const int n0 = blockIdx.y * 16;        // grid.y: block of 16 weight rows
    if (n0 >= p.n_rows(ctx)) return;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int kq = lane >> 4;  // which 8-element quarter of a 32-wide k step
    const int steps = p.k_steps(ctx);
    const int s_begin = wave * steps / KS;
    const int s_end = (wave + 1) * steps / KS;

    const typename P::RowW wrow = p.row_w(ctx, n0 + (lane & 15));
    const typename P::RowX xrow = p.row_x(ctx, lane & 15);

    f32x4 acc[NMAT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m) acc[m] = f32x4{};

    constexpr int kBatch = 8;
    for (int s0 = s_begin; s0 < s_end; s0 += kBatch) {
        uint4 wa[NMAT][kBatch];
        typename P::XFrag xb[kBatch];
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
            if (s0 + i < s_end) {
#pragma unroll
                for (int m = 0; m < NMAT; ++m) wa[m][i] = p.load_w(ctx, wrow, m, s0 + i, kq);
                xb[i] = p.load_x(ctx, xrow, s0 + i, kq);
            }
        }
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
            if (s0 + i < s_end) {
#pragma unroll
                for (int m = 0; m < NMAT; ++m) acc[m] = P::mma(acc[m], wa[m][i], xb[i]);
            }
        }
    }

#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wave][m][(4 * (lane >> 4) + r) * 16 + (lane & 15)] = acc[m][r];
    __syncthreads();
    if (threadIdx.x < 256) {
        const int i = threadIdx.x >> 4;
        const int j = threadIdx.x & 15;
        float v[NMAT];
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
            float s = 0.f;
#pragma unroll
            for (int w = 0; w < KS; ++w) s += red[w][m][threadIdx.x];
            v[m] = s;
        }
        p.epilogue(ctx, n0 + i, j, v);
    }
}

}  // namespace lmoe
