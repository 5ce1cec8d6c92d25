// Expert work of a small batch (decode / speculative verify, T <= 16 tokens) in two launches
// with no dependency between workgroups inside either launch.
//
// 1. Gate/up (decode_gu_kernel).  A work item is (tile, block): the tile's tokens (<= 16 rows of
//    one segment) and 16 consecutive columns f of the SwiGLU width; a wave computes the gate and
//    up rows of the block against the tokens (K = latent, weights streamed from HBM, double
//    buffered) and stores SiLU(g) * u as bf16 into
//        H[segment row][f].
//    Items are dealt evenly over the compute units, so every CU streams the same share.
// 2. Down and merge (decode_dc_kernel).  A workgroup owns 16 latent rows and one group of the
//    work list (the tiles are split into G contiguous groups).  Its waves take the group's tiles
//    in turn; for a tile, Y = H(tile rows) . down^T over the full SwiGLU width (weights streamed,
//    H rows read back from L2), and each row's result is added, times its routing weight (1 for
//    the shared expert), to the wave's per-token accumulator in LDS.  The waves' accumulators are
//    then summed in wave order and written as the group's partial merged rows
//        mpart[g][t][latent]  (fp32).
//    The U projection sums the G partials (in group order) while staging its input.
//
// Every sum runs in a fixed order (tiles in work-list order within a wave, waves in order,
// groups in order), so results do not depend on scheduling.
#pragma once

#include "gemm_stream.hpp"
#include "problems.hpp"

namespace lmoe {

template <bool MX>
struct DecodeExperts {
    SegSpace seg;
    const uint16_t* z16;  // [T][L]
    const void* experts;
    size_t rec_bytes;
    const uint16_t* shared;
    int L, F, Fs, Hs;  // Hs = max(F, Fs): row pitch of H
    int nblocks;       // 16-row blocks of the widest segment: ceil(Hs / 16)
    uint16_t* H;       // [T*k + T][Hs] bf16, segment-row order
    const float* w;    // [T][k] routing weights (slot order)
    float* mpart;      // [G][T][L]
    int groups;        // G
};

// ---- gate/up ----------------------------------------------------------------------------------
template <int W, int CH, bool MXR, bool MX>
__device__ __forceinline__ void gu_item(const DecodeExperts<MX>& d, const Tile& tl, int f0,
                                        const typename ExpertRows<MX>::Mat (&mats)[3]) {
    using ER = ExpertRows<MX>;
    constexpr int SPL = ER::kSPL;
    const int lane = threadIdx.x & 63;
    const int kq = lane >> 4;
    const int j = lane & 15;
    const int L = d.L;
    const int nrows = tl.nrows;
    const typename ER::Row rg = ER::row(mats[0], f0 + j, L), ru = ER::row(mats[1], f0 + j, L);
    const int tok = d.seg.token_of(tl.seg, tl.row0 + min(j, nrows - 1));
    const uint16_t* xr = d.z16 + (size_t)tok * L;
    const bool xok = j < nrows;
    const int groups = L / (32 * SPL);
    const int nch = (groups + CH - 1) / CH;
    f32x4 ag = f32x4{}, au = f32x4{};
    typename ER::WRaw ga[CH], ua[CH], gbuf[CH], ubuf[CH];
    uint4 xa[CH * SPL], xb[CH * SPL];
    auto load = [&](typename ER::WRaw (&g)[CH], typename ER::WRaw (&u)[CH], uint4 (&x)[CH * SPL], int c) {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int gi = min(c * CH + i, groups - 1);
            g[i] = ER::template load<MXR>(rg, gi, kq);
            u[i] = ER::template load<MXR>(ru, gi, kq);
#pragma unroll
            for (int t = 0; t < SPL; ++t) x[i * SPL + t] = ld16(xr + step_k<SPL>(gi * SPL + t, kq));
        }
    };
    auto compute = [&](const typename ER::WRaw (&g)[CH], const typename ER::WRaw (&u)[CH], const uint4 (&x)[CH * SPL],
                       int c) {
#pragma unroll
        for (int i = 0; i < CH; ++i)
            if (c * CH + i < groups)
#pragma unroll
                for (int t = 0; t < SPL; ++t) {
                    const uint4 xv = sel4(xok, x[i * SPL + t]);
                    ag = mfma16(ER::template frag<MXR>(g[i], t), xv, ag);
                    au = mfma16(ER::template frag<MXR>(u[i], t), xv, au);
                }
    };
    load(ga, ua, xa, 0);
    for (int c = 0; c < nch; c += 2) {
        load(gbuf, ubuf, xb, c + 1);
        compute(ga, ua, xa, c);
        load(ga, ua, xa, c + 2);
        if (c + 1 < nch) compute(gbuf, ubuf, xb, c + 1);
    }
    // this lane holds f rows f0 + 4 kq + r (r = 0..3) of segment row j
    if (xok) {
        const uint2 v = make_uint2(pack_bf2(silu(ag[0]) * au[0], silu(ag[1]) * au[1]),
                                   pack_bf2(silu(ag[2]) * au[2], silu(ag[3]) * au[3]));
        *reinterpret_cast<uint2*>(d.H + (size_t)(tl.row0 + j) * d.Hs + f0 + 4 * kq) = v;
    }
}

// Gate/up work items are (tile, 16-row block of the SwiGLU width), in work-list order with the
// blocks of a tile adjacent.  The grid holds one workgroup per compute unit (W waves, at most
// one such workgroup fits a CU) and item i goes to workgroup i % grid, wave (i / grid) % W, so
// every CU streams the same number of items; blocks past the segment's width are skipped.
template <int W, int CH, bool MX>
__global__ __launch_bounds__(64 * W) void decode_gu_kernel(const DecodeExperts<MX> d) {
    const int wave = threadIdx.x >> 6;
    const int nitems = *d.seg.ntiles * d.nblocks;
    for (int item = blockIdx.x + gridDim.x * wave; item < nitems; item += gridDim.x * W) {
        const int tile = item / d.nblocks, blk = item - tile * d.nblocks;
        const Tile tl = d.seg.tiles[tile];
        typename ExpertRows<MX>::Mat mats[3];
        int Fseg;
        bool mx;
        segment_mats<MX>(d.experts, d.rec_bytes, d.shared, tl.seg, d.seg.E, d.F, d.Fs, d.L, mats, Fseg, mx);
        const int f0 = blk * 16;
        if (f0 >= Fseg) continue;  // widths are multiples of 16
        if (mx)
            gu_item<W, CH, MX, MX>(d, tl, f0, mats);
        else
            gu_item<W, CH, false, MX>(d, tl, f0, mats);
    }
}

// ---- down + merge -----------------------------------------------------------------------------
// One tile: acc = down(latent rows n0 .. n0 + 15) . H(tile rows)^T over K = Fseg.
template <int CH, bool MXR, bool MX>
__device__ __forceinline__ f32x4 dc_tile(const DecodeExperts<MX>& d, const Tile& tl,
                                         const typename ExpertRows<MX>::Mat& down, int Fseg, int n0) {
    using ER = ExpertRows<MX>;
    constexpr int SPL = ER::kSPL;
    const int lane = threadIdx.x & 63;
    const int kq = lane >> 4;
    const int j = lane & 15;
    const int nrows = tl.nrows;
    const typename ER::Row rw = ER::row(down, n0 + j, Fseg);
    const uint16_t* hr = d.H + (size_t)(tl.row0 + min(j, nrows - 1)) * d.Hs;
    const bool ok = j < nrows;
    const int groups = Fseg / (32 * SPL);
    const int nch = (groups + CH - 1) / CH;
    f32x4 acc = f32x4{};
    typename ER::WRaw wa[CH], wb[CH];
    uint4 ha[CH * SPL], hb[CH * SPL];
    auto load = [&](typename ER::WRaw (&w)[CH], uint4 (&h)[CH * SPL], int c) {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int gi = min(c * CH + i, groups - 1);
            w[i] = ER::template load<MXR>(rw, gi, kq);
#pragma unroll
            for (int t = 0; t < SPL; ++t) h[i * SPL + t] = ld16(hr + step_k<SPL>(gi * SPL + t, kq));
        }
    };
    auto compute = [&](const typename ER::WRaw (&w)[CH], const uint4 (&h)[CH * SPL], int c) {
#pragma unroll
        for (int i = 0; i < CH; ++i)
            if (c * CH + i < groups)
#pragma unroll
                for (int t = 0; t < SPL; ++t) acc = mfma16(ER::template frag<MXR>(w[i], t), sel4(ok, h[i * SPL + t]), acc);
    };
    load(wa, ha, 0);
    for (int c = 0; c < nch; c += 2) {
        load(wb, hb, c + 1);
        compute(wa, ha, c);
        load(wa, ha, c + 2);
        if (c + 1 < nch) compute(wb, hb, c + 1);
    }
    return acc;
}

// grid (L / 16, G); W waves.  Every wave must reach the barrier (no early return).
template <int W, int CH, bool MX>
__global__ __launch_bounds__(64 * W) void decode_dc_kernel(const DecodeExperts<MX> d) {
    __shared__ float macc[W][16][17];  // per wave: [token][latent row of the block] (+1 pad)
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int kq = lane >> 4, j = lane & 15;
    const int n0 = blockIdx.x * 16, grp = blockIdx.y;
    const int T = d.seg.T, k = d.seg.k, E = d.seg.E;
    const int nt = *d.seg.ntiles;
    const int tb = (int)((long)grp * nt / d.groups), te = (int)((long)(grp + 1) * nt / d.groups);
    for (int i = lane; i < 16 * 17; i += 64) (&macc[wave][0][0])[i] = 0.f;
    // the accumulator is private to the wave (a wave's LDS accesses complete in order)
    for (int ti = tb + wave; ti < te; ti += W) {
        const Tile tl = d.seg.tiles[ti];
        typename ExpertRows<MX>::Mat mats[3];
        int Fseg;
        bool mx;
        segment_mats<MX>(d.experts, d.rec_bytes, d.shared, tl.seg, E, d.F, d.Fs, d.L, mats, Fseg, mx);
        const f32x4 acc = mx ? dc_tile<CH, MX, MX>(d, tl, mats[2], Fseg, n0) : dc_tile<CH, false, MX>(d, tl, mats[2], Fseg, n0);
        // lane (kq, j): latent rows n0 + 4 kq + r of segment row j -> its token and weight
        if (j < tl.nrows) {
            const int p = tl.row0 + j;
            int t = -1;
            float wt = 0.f;
            if (tl.seg == E) {
                t = p - T * k;
                wt = 1.f;
            } else {
                const int f = d.seg.perm[p];
                if (f >= 0) {
                    t = f / k;
                    wt = d.w[f];
                }
            }
            if (t >= 0)
#pragma unroll
                for (int r = 0; r < 4; ++r) macc[wave][t][4 * kq + r] += wt * acc[r];
        }
    }
    __syncthreads();
    // thread e: token e / 16, latent row n0 + e % 16; the waves' sums in wave order
    for (int e = threadIdx.x; e < 256; e += 64 * W) {
        const int t = e >> 4, r = e & 15;
        if (t < T) {
            float s = 0.f;
#pragma unroll
            for (int w = 0; w < W; ++w) s += macc[w][t][r];
            d.mpart[((size_t)grp * T + t) * d.L + n0 + r] = s;
        }
    }
}

}  // namespace lmoe
