// Weight-streaming bf16 MFMA kernel for small token batches (decode / speculative verify):
// C[n][t] = sum_k W[n][k] * X[t][k] for blocks of 16 weight rows n and up to 16 tokens t.
//
// At a handful of tokens the work is bound by reading every weight once from HBM, so the
// weights are the MFMA A operand, loaded straight from global memory into registers in the
// v_mfma_f32_16x16x32_bf16 operand layout, and the tokens are the B operand (columns beyond
// the batch are zero).  A workgroup has WAVES waves; each block of 16 weight rows is shared
// by KS waves that split K into contiguous slices and sum their 16x16 partial tiles in LDS in
// slice order (deterministic), so a workgroup covers WAVES/KS row blocks.  Weight loads are
// double buffered in batches of BATCH MFMA steps so every wave keeps two batches in flight.
//
// The token operand is either staged once per workgroup in LDS (P::kXLds; rows padded by 16
// bytes so the 16 token rows of a fragment read fall in different banks) or read from global
// memory (L2-resident) per step.
//
// A problem type P supplies the tile mapping, weight-row addressing and loads (kSPL MFMA steps
// per weight load: 1 for bf16, 4 for MXFP4 where a lane reads 16 bytes = 32 values and one
// scale), the k order of a step (step_k, shared by both operands so the dot product covers
// every k exactly once), and the epilogue.
#pragma once

#include "common.hpp"

namespace lmoe {

// k offset of the 8 values an MFMA step reads, per weight-load granularity.
template <int SPL>
__device__ __forceinline__ int step_k(int s, int kq) {
    if constexpr (SPL == 1) {
        return s * 32 + kq * 8;
    } else {
        static_assert(SPL == 4, "1 or 4 steps per load");
        return (s >> 2) * 128 + kq * 32 + (s & 3) * 8;
    }
}

template <int WAVES, int KS, int NMAT, int BATCH, class P>
__global__ __launch_bounds__(64 * WAVES) void stream_gemm_kernel(const P p) {
    static_assert(WAVES % KS == 0, "whole row blocks per workgroup");
    static_assert(BATCH % P::kSPL == 0, "batches hold whole weight loads");
    constexpr int RBW = WAVES / KS;          // row blocks per workgroup
    constexpr int GB = BATCH / P::kSPL;      // weight loads per batch and matrix
    extern __shared__ uint4 lds_x[];
    __shared__ float red[KS > 1 ? WAVES : 1][KS > 1 ? NMAT : 1][KS > 1 ? 256 : 1];

    typename P::Ctx ctx;
    if (!p.tile(blockIdx.x, ctx)) return;  // grid.x: token tile / work-list entry
    const int nrows = p.n_rows(ctx);
    if (blockIdx.y * RBW * 16 >= nrows) return;  // grid.y: groups of RBW row blocks

    if constexpr (P::kXLds) {
        p.stage_x(ctx, reinterpret_cast<uint8_t*>(lds_x));
        __syncthreads();
    }
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int kq = lane >> 4;
    const int j = lane & 15;
    const int n0 = (blockIdx.y * RBW + wave / KS) * 16;
    const int slice = wave % KS;
    const int groups = p.k_steps(ctx) / P::kSPL;
    const int g_begin = slice * groups / KS;
    const int g_end = (slice + 1) * groups / KS;

    const typename P::RowW wrow = p.row_w(ctx, n0 + j);
    const typename P::RowX xrow = p.row_x(ctx, j);

    f32x4 acc[NMAT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m) acc[m] = f32x4{};

    typename P::WRaw cur[NMAT][GB], nxt[NMAT][GB];
    auto load = [&](typename P::WRaw (&dst)[NMAT][GB], int g0) {
#pragma unroll
        for (int gi = 0; gi < GB; ++gi)
            if (g0 + gi < g_end)
#pragma unroll
                for (int m = 0; m < NMAT; ++m) dst[m][gi] = p.load_w(ctx, wrow, m, g0 + gi, kq);
    };
    if (g_begin < g_end) load(cur, g_begin);
    for (int g0 = g_begin; g0 < g_end; g0 += GB) {
        const bool more = g0 + GB < g_end;
        if (more) load(nxt, g0 + GB);
#pragma unroll
        for (int gi = 0; gi < GB; ++gi) {
            if (g0 + gi < g_end) {
#pragma unroll
                for (int t = 0; t < P::kSPL; ++t) {
                    const int s = (g0 + gi) * P::kSPL + t;
                    typename P::XFrag xb;
                    if constexpr (P::kXLds)
                        xb = p.lds_frag(ctx, reinterpret_cast<const uint8_t*>(lds_x), j, step_k<P::kSPL>(s, kq));
                    else
                        xb = p.load_x(ctx, xrow, step_k<P::kSPL>(s, kq));
#pragma unroll
                    for (int m = 0; m < NMAT; ++m) acc[m] = P::mma(acc[m], p.wfrag_ctx(ctx, cur[m][gi], t), xb);
                }
            }
        }
        if (more) {
#pragma unroll
            for (int gi = 0; gi < GB; ++gi)
#pragma unroll
                for (int m = 0; m < NMAT; ++m) cur[m][gi] = nxt[m][gi];
        }
    }

    if constexpr (KS == 1) {
        if (n0 < nrows) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float v[NMAT];
#pragma unroll
                for (int m = 0; m < NMAT; ++m) v[m] = acc[m][r];
                p.epilogue(ctx, n0 + 4 * kq + r, j, v);
            }
        }
    } else {
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[wave][m][(4 * kq + r) * 16 + j] = acc[m][r];
        __syncthreads();
        for (int e = threadIdx.x; e < RBW * 256; e += 64 * WAVES) {
            const int rb = e >> 8, el = e & 255;
            const int nb = (blockIdx.y * RBW + rb) * 16;
            if (nb >= nrows) continue;
            float v[NMAT];
#pragma unroll
            for (int m = 0; m < NMAT; ++m) {
                float sum = 0.f;
#pragma unroll
                for (int sl = 0; sl < KS; ++sl) sum += red[rb * KS + sl][m][el];
                v[m] = sum;
            }
            p.epilogue(ctx, nb + (el >> 4), el & 15, v);
        }
    }
}

}  // namespace lmoe
