// Weight-streaming bf16 MFMA kernel for small token batches (decode / speculative verify):
// C[n][t] = sum_k W[n][k] * X[t][k] for blocks of 16 weight rows n and up to 16 tokens t.
//
// At a handful of tokens the work is bound by reading every weight once from HBM, so the
// weights are the MFMA A operand, loaded straight from global memory into registers in the
// v_mfma_f32_16x16x32_bf16 operand layout, and the tokens are the B operand (columns beyond
// the batch are zero), loaded from global memory (they stay L2-resident).
//
// Work items are (tile, group of WAVES/KS row blocks); a persistent grid walks them, so a work
// list produced on the device needs no empty workgroups.  Inside an item each 16-row block is
// shared by KS waves that split K into contiguous slices; a wave streams its slice in chunks of
// CH weight loads per matrix, double buffered: the next chunk's loads are in flight while the
// current chunk feeds the MFMAs.  Loads are branch-free (rows past the matrix and chunks past
// the slice are clamped to valid addresses; their results are discarded), so the compiler can
// keep exact wait counts.  The KS partial 16x16 tiles of a row block are summed in LDS in slice
// order (deterministic).
//
// A problem type P supplies the tile mapping, weight-row addressing and loads (kSPL MFMA steps
// per weight load: 1 for bf16, 4 for MXFP4 where a lane reads 16 bytes = 32 values and one
// scale), the k order of a step (step_k, shared by both operands so the dot product covers
// every k exactly once), and the epilogue.  Problems whose rows may be MXFP4 or bf16 within one
// launch (P::kMixed) pick the row format once per work item.
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

template <int WAVES, int KS, int NMAT, int CH, bool MXR, class P>
__device__ __forceinline__ void stream_item(const P& p, const typename P::Ctx& ctx, int rg, int nrows,
                                            float (*red)[256]) {
    constexpr int RBW = WAVES / KS;
    constexpr int SPL = P::kSPL;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int kq = lane >> 4;
    const int j = lane & 15;
    const int n0 = (rg * RBW + wave / KS) * 16;
    const int slice = wave % KS;
    const int groups = p.k_steps(ctx) / SPL;
    const int g_begin = slice * groups / KS;
    const int g_end = (slice + 1) * groups / KS;
    const int nch = (g_end - g_begin + CH - 1) / CH;
    const typename P::RowW wrow = p.row_w(ctx, min(n0 + j, nrows - 1));
    const typename P::XRow xrow = p.x_row(ctx, j);

    f32x4 acc[NMAT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m) acc[m] = f32x4{};

    typename P::WRaw wa[NMAT][CH], wb[NMAT][CH];
    typename P::XRaw xa[CH * SPL], xb[CH * SPL];
    auto load = [&](typename P::WRaw (&w)[NMAT][CH], typename P::XRaw (&x)[CH * SPL], int c) {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int g = min(g_begin + c * CH + i, g_end - 1);
#pragma unroll
            for (int m = 0; m < NMAT; ++m) w[m][i] = p.template load_w<MXR>(ctx, wrow, m, g, kq);
#pragma unroll
            for (int t = 0; t < SPL; ++t) x[i * SPL + t] = p.load_x(ctx, xrow, step_k<SPL>(g * SPL + t, kq));
        }
    };
    auto compute = [&](const typename P::WRaw (&w)[NMAT][CH], const typename P::XRaw (&x)[CH * SPL], int c) {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            if (g_begin + c * CH + i < g_end) {
#pragma unroll
                for (int t = 0; t < SPL; ++t) {
                    const typename P::XFrag xv = p.x_frag(xrow, x[i * SPL + t]);
#pragma unroll
                    for (int m = 0; m < NMAT; ++m) acc[m] = P::mma(acc[m], P::template wfrag<MXR>(w[m][i], t), xv);
                }
            }
        }
    };
    if (nch > 0) {
        load(wa, xa, 0);
        for (int c = 0; c < nch; c += 2) {
            load(wb, xb, c + 1);
            compute(wa, xa, c);
            load(wa, xa, c + 2);
            if (c + 1 < nch) compute(wb, xb, c + 1);
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
            for (int r = 0; r < 4; ++r) red[wave * NMAT + m][(4 * kq + r) * 16 + j] = acc[m][r];
        __syncthreads();
        for (int e = threadIdx.x; e < RBW * 256; e += 64 * WAVES) {
            const int rb = e >> 8, el = e & 255;
            const int nb = (rg * RBW + rb) * 16;
            if (nb >= nrows) continue;
            float v[NMAT];
#pragma unroll
            for (int m = 0; m < NMAT; ++m) {
                float sum = 0.f;
#pragma unroll
                for (int sl = 0; sl < KS; ++sl) sum += red[(rb * KS + sl) * NMAT + m][el];
                v[m] = sum;
            }
            p.epilogue(ctx, nb + (el >> 4), el & 15, v);
        }
        __syncthreads();  // red is reused by the next item
    }
}

// grid.x workgroups walk items (tile, row group) with a stride; `rgroups` row groups per tile.
template <int WAVES, int KS, int NMAT, int CH, class P>
__global__ __launch_bounds__(64 * WAVES) void stream_gemm_kernel(const P p, int rgroups) {
    static_assert(WAVES % KS == 0, "whole row blocks per workgroup");
    constexpr int RBW = WAVES / KS;
    __shared__ float red[KS > 1 ? WAVES * NMAT : 1][256];
    const int nitems = p.num_tiles() * rgroups;
    for (int item = blockIdx.x; item < nitems; item += gridDim.x) {
        const int tile = item / rgroups, rg = item - tile * rgroups;
        typename P::Ctx ctx;
        p.tile(tile, ctx);
        const int nrows = p.n_rows(ctx);
        if (rg * RBW * 16 >= nrows) continue;
        if constexpr (P::kMixed) {
            if (p.mx_rows(ctx))
                stream_item<WAVES, KS, NMAT, CH, true>(p, ctx, rg, nrows, red);
            else
                stream_item<WAVES, KS, NMAT, CH, false>(p, ctx, rg, nrows, red);
        } else {
            stream_item<WAVES, KS, NMAT, CH, false>(p, ctx, rg, nrows, red);
        }
    }
}

}  // namespace lmoe
