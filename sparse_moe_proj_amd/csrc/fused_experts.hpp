// All expert work of a small batch in one persistent launch: SwiGLU gate/up of every segment,
// then the down projections, then the weighted merge, with device-side dependencies instead of
// kernel boundaries.
//
//  * The grid never exceeds the number of workgroups that fit on the GPU at once, so every
//    workgroup a wait depends on is running.
//  * Phase 1 walks the gate/up items (tile, row group); finishing one increments the tile's
//    counter with release semantics.
//  * Phase 2 walks the down items: a wave first issues the loads of its whole slice of down
//    weights (they do not depend on H), then one thread waits (acquire) until every gate/up item
//    of the tile is done, then the tile's H rows are read and multiplied.  The waits are bounded:
//    a wait that runs out sets *status and the workgroup carries on (results are then invalid;
//    this can only happen when other work holds the compute units).
//  * Each down row group has an arrival counter; the workgroup that completes a row group's last
//    tile merges that block of latent columns for every token in fixed slot order:
//    m[t] = Y[shared t] + sum_s w[t][s] * Y[t k + s]  (bf16 out).
// Counters and *status are zeroed by the permutation kernel that precedes this launch.
#pragma once

#include "gemm_stream.hpp"
#include "problems.hpp"

namespace lmoe {

template <bool MX>
struct FusedExperts {
    StreamUp<MX> up;
    StreamDown<MX> dn;
    int up_rg;          // gate/up row groups per tile
    int dn_rg;          // down row groups per tile
    int32_t* up_done;   // [max tiles]
    int32_t* dn_done;   // [dn_rg]
    int32_t* status;    // wait timeout flag
    const float* w;     // [T][k] routing weights
    int T, k, has_shared;
    uint16_t* m16;      // [T][L] merged latent (bf16)
};

constexpr int kSpinLimit = 1 << 18;

__device__ __forceinline__ void wait_count(const int32_t* cnt, int target, int32_t* status) {
    int polls = 0;
    while (__hip_atomic_load(cnt, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) < target) {
        __builtin_amdgcn_s_sleep(2);
        if (++polls > kSpinLimit) {
            atomicOr(status, 1);
            break;
        }
    }
}

// Down item: burst-load the weight slice, wait for the tile's gate/up items, then compute.
template <int WAVES, int MAXG, bool MXR, bool MX>
__device__ __forceinline__ void down_item(const FusedExperts<MX>& f, const typename StreamDown<MX>::Ctx& ctx, int tile,
                                          int rg) {
    using P = StreamDown<MX>;
    constexpr int SPL = P::kSPL;
    const P& p = f.dn;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int kq = lane >> 4;
    const int j = lane & 15;
    const int nrows = p.n_rows(ctx);
    const int n0 = (rg * WAVES + wave) * 16;
    const int groups = p.k_steps(ctx) / SPL;
    const typename P::RowW wrow = p.row_w(ctx, min(n0 + j, nrows - 1));

    typename P::WRaw wv[MAXG];
#pragma unroll
    for (int i = 0; i < MAXG; ++i) wv[i] = p.template load_w<MXR>(ctx, wrow, 0, min(i, groups - 1), kq);

    // the tile's H rows exist once all its gate/up row groups are done
    const int need = (f.up.n_rows_for(ctx.seg) + 16 * WAVES - 1) / (16 * WAVES);
    if (threadIdx.x == 0) wait_count(f.up_done + tile, need, f.status);
    __syncthreads();

    const typename P::XRow xrow = p.x_row(ctx, j);
    f32x4 acc = f32x4{};
    for (int c0 = 0; c0 < groups; c0 += MAXG) {
        if (c0 > 0) {
#pragma unroll
            for (int i = 0; i < MAXG; ++i) wv[i] = p.template load_w<MXR>(ctx, wrow, 0, min(c0 + i, groups - 1), kq);
        }
        typename P::XRaw xv[MAXG * SPL];
#pragma unroll
        for (int i = 0; i < MAXG; ++i)
#pragma unroll
            for (int t = 0; t < SPL; ++t)
                xv[i * SPL + t] = p.load_x(ctx, xrow, step_k<SPL>(min(c0 + i, groups - 1) * SPL + t, kq));
#pragma unroll
        for (int i = 0; i < MAXG; ++i)
            if (c0 + i < groups)
#pragma unroll
                for (int t = 0; t < SPL; ++t)
                    acc = P::mma(acc, P::template wfrag<MXR>(wv[i], t), p.x_frag(xrow, xv[i * SPL + t]));
    }
    if (n0 < nrows) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float v[1] = {acc[r]};
            p.epilogue(ctx, n0 + 4 * kq + r, j, v);
        }
    }
}

template <int WAVES, int CH, int MAXG, bool MX>
__global__ __launch_bounds__(64 * WAVES) void fused_experts_kernel(const FusedExperts<MX> f) {
    __shared__ int s_last;
    const int ntiles = f.up.num_tiles();

    // phase 1: gate/up
    const int n_up = ntiles * f.up_rg;
    for (int item = blockIdx.x; item < n_up; item += gridDim.x) {
        const int tile = item / f.up_rg, rg = item - tile * f.up_rg;
        typename StreamUp<MX>::Ctx ctx;
        f.up.tile(tile, ctx);
        const int nrows = f.up.n_rows(ctx);
        if (rg * WAVES * 16 >= nrows) continue;
        if (f.up.mx_rows(ctx))
            stream_item<WAVES, 1, 2, CH, MX>(f.up, ctx, rg, nrows, nullptr);
        else
            stream_item<WAVES, 1, 2, CH, false>(f.up, ctx, rg, nrows, nullptr);
        __syncthreads();
        if (threadIdx.x == 0) __hip_atomic_fetch_add(f.up_done + tile, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }

    // phase 2: down + merge
    const int n_dn = ntiles * f.dn_rg;
    const int L = f.dn.L;
    for (int item = blockIdx.x; item < n_dn; item += gridDim.x) {
        const int tile = item / f.dn_rg, rg = item - tile * f.dn_rg;
        typename StreamDown<MX>::Ctx ctx;
        f.dn.tile(tile, ctx);
        if (f.dn.mx_rows(ctx))
            down_item<WAVES, MAXG, MX, MX>(f, ctx, tile, rg);
        else
            down_item<WAVES, MAXG, false, MX>(f, ctx, tile, rg);
        __syncthreads();
        if (threadIdx.x == 0) {
            const int old = __hip_atomic_fetch_add(f.dn_done + rg, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
            s_last = old == ntiles - 1;
        }
        __syncthreads();
        if (s_last) {
            // merge latent columns [c0, c0 + 16 * WAVES) of every token
            const int c0 = rg * WAVES * 16;
            const int ncols = min(16 * WAVES, L - c0);
            for (int e = threadIdx.x; e < f.T * ncols; e += blockDim.x) {
                const int t = e / ncols, c = c0 + (e - t * ncols);
                float acc = f.has_shared ? f.dn.Y[((size_t)f.T * f.k + t) * L + c] : 0.f;
                for (int s = 0; s < f.k; ++s) acc += f.w[t * f.k + s] * f.dn.Y[((size_t)t * f.k + s) * L + c];
                f.m16[(size_t)t * L + c] = (uint16_t)f2bf(acc);
            }
        }
    }
}

}  // namespace lmoe
