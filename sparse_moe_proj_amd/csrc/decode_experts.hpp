// All expert work of a small batch (decode / speculative verify) in one launch with no
// dependency between workgroups, followed by a small merge launch.
//
// A work item is (tile, slice): the tile's tokens (<= 16 rows of one segment) and FS consecutive
// columns f of the SwiGLU width.  The workgroup computes the gate and up rows f = slice * FS ..
// + FS against the tokens (K = latent; weights streamed from HBM, double buffered, 16 rows per
// wave or per group of waves splitting K), applies SiLU(g) * u in registers and stores the H
// slice (bf16) in LDS.  The
// workgroup then multiplies that H slice by the same FS columns of the down matrix (a contiguous
// chunk of every latent row) and writes the partial product
//     P[dest row][slice][latent]  (fp32),
// the destination row being token-major (t*k + s for routed rows, T*k + t for the shared expert).
// The merge sums the slices of a row in slice order, so results do not depend on scheduling:
//     m[t] = sum_q P[T*k + t][q] + sum_s w[t][s] * sum_q P[t*k + s][q].
//
// Splitting the down projection over slices of F costs one fp32 partial row of the latent width
// per (token, slot, slice), a few MB at decode sizes, and removes the kernel boundary between the
// gate/up and the down projections without any wait between workgroups.
#pragma once

#include "gemm_stream.hpp"
#include "problems.hpp"

#ifndef LMOE_DECODE_RB
#define LMOE_DECODE_RB 4
#endif

namespace lmoe {

template <bool MX>
struct DecodeExperts {
    SegSpace seg;
    const uint16_t* z16;  // [T][L]
    const void* experts;
    size_t rec_bytes;
    const uint16_t* shared;
    int L, F, Fs, nslices;  // nslices = max(F, Fs) / slice width
    float* P;               // [R][nslices][L]
};

// WAVES waves per item; KSU waves share each 16-row block of the gate/up phase, splitting K
// (their partial sums meet in LDS, summed in wave order); FS = 16 * WAVES / KSU columns per slice.
template <int WAVES, int KSU>
struct DecodeShape {
    static_assert(WAVES % KSU == 0, "whole row blocks per item");
    static constexpr int kFB = WAVES / KSU;  // 16-row blocks of F per item
    static constexpr int kFS = 16 * kFB;     // slice width
    static constexpr int kHP = kFS + 8;      // LDS row pitch (elements) of the H slice; 16-byte multiple
    static constexpr int kRed = KSU > 1 ? WAVES * 2 * 4 * 64 : 1;  // partial gate/up sums (floats)
};

template <int WAVES, int KSU, int CH, bool MXR, bool MX>
__device__ __forceinline__ void decode_item(const DecodeExperts<MX>& d, const Tile& tl, int slice,
                                            const typename ExpertRows<MX>::Mat (&mats)[3], int Fseg, uint16_t* Hs,
                                            float* red) {
    using ER = ExpertRows<MX>;
    using DS = DecodeShape<WAVES, KSU>;
    constexpr int SPL = ER::kSPL;
    constexpr int FS = DS::kFS;
    constexpr int HP = DS::kHP;
    static_assert(FS % (32 * SPL) == 0, "a slice holds whole weight loads");
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int kq = lane >> 4;
    const int j = lane & 15;
    const int L = d.L;
    const int nrows = tl.nrows;

    // down-phase geometry (its first weight batch is requested before the gate/up results exist)
    constexpr int KG = FS / (32 * SPL);  // weight loads per row and slice
    constexpr int RB = LMOE_DECODE_RB;   // row blocks per load batch
    const int nblk = L / 16;
    const int g0 = slice * KG;
    const int nmine = (nblk - wave + WAVES - 1) / WAVES;  // row blocks wave, wave + WAVES, ...
    typename ER::WRaw wa[RB][KG], wb[RB][KG];
    auto load_dn = [&](typename ER::WRaw (&w)[RB][KG], int b0) {
#pragma unroll
        for (int i = 0; i < RB; ++i) {
            const int blk = wave + WAVES * min(b0 + i, nmine - 1);
            const typename ER::Row rw = ER::row(mats[2], blk * 16 + j, Fseg);
#pragma unroll
            for (int g = 0; g < KG; ++g) w[i][g] = ER::template load<MXR>(rw, g0 + g, kq);
        }
    };

    // ---- gate/up: rows f of block wave / KSU, K range `half` of KSU
    {
        const int fb = wave / KSU, half = wave % KSU;
        const int f = slice * FS + fb * 16 + j;  // < Fseg: Fseg is a multiple of FS
        const typename ER::Row rg = ER::row(mats[0], f, L), ru = ER::row(mats[1], f, L);
        const int tok = d.seg.token_of(tl.seg, tl.row0 + min(j, nrows - 1));
        const uint16_t* xr = d.z16 + (size_t)tok * L;
        const bool xok = j < nrows;
        const int groups = L / (32 * SPL);
        const int gb = half * groups / KSU, ge = (half + 1) * groups / KSU;
        const int nch = (ge - gb + CH - 1) / CH;
        f32x4 ag = f32x4{}, au = f32x4{};
        typename ER::WRaw ga[CH], ua[CH], gbuf[CH], ubuf[CH];
        uint4 xa[CH * SPL], xb[CH * SPL];
        auto load = [&](typename ER::WRaw (&g)[CH], typename ER::WRaw (&u)[CH], uint4 (&x)[CH * SPL], int c) {
#pragma unroll
            for (int i = 0; i < CH; ++i) {
                const int gi = min(gb + c * CH + i, ge - 1);
                g[i] = ER::template load<MXR>(rg, gi, kq);
                u[i] = ER::template load<MXR>(ru, gi, kq);
#pragma unroll
                for (int t = 0; t < SPL; ++t) x[i * SPL + t] = ld16(xr + step_k<SPL>(gi * SPL + t, kq));
            }
        };
        auto compute = [&](const typename ER::WRaw (&g)[CH], const typename ER::WRaw (&u)[CH],
                           const uint4 (&x)[CH * SPL], int c) {
#pragma unroll
            for (int i = 0; i < CH; ++i)
                if (gb + c * CH + i < ge)
#pragma unroll
                    for (int t = 0; t < SPL; ++t) {
                        const uint4 xv = sel4(xok, x[i * SPL + t]);
                        ag = mfma16(ER::template frag<MXR>(g[i], t), xv, ag);
                        au = mfma16(ER::template frag<MXR>(u[i], t), xv, au);
                    }
        };
        if (nch > 0) {
            load(ga, ua, xa, 0);
            for (int c = 0; c < nch; c += 2) {
                load(gbuf, ubuf, xb, c + 1);
                compute(ga, ua, xa, c);
                load(ga, ua, xa, c + 2);
                if (c + 1 < nch) compute(gbuf, ubuf, xb, c + 1);
            }
        }
        if (nmine > 0) load_dn(wa, 0);
        // this lane holds f rows 4 kq + r (of the block's 16) for token column j
        if constexpr (KSU > 1) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                red[((wave * 2 + 0) * 4 + r) * 64 + lane] = ag[r];
                red[((wave * 2 + 1) * 4 + r) * 64 + lane] = au[r];
            }
            __syncthreads();
            if (half == 0) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float g = 0.f, u = 0.f;
#pragma unroll
                    for (int h = 0; h < KSU; ++h) {
                        g += red[(((wave + h) * 2 + 0) * 4 + r) * 64 + lane];
                        u += red[(((wave + h) * 2 + 1) * 4 + r) * 64 + lane];
                    }
                    Hs[j * HP + fb * 16 + 4 * kq + r] = (uint16_t)(xok ? f2bf(silu(g) * u) : 0u);
                }
            }
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                Hs[j * HP + fb * 16 + 4 * kq + r] = (uint16_t)(xok ? f2bf(silu(ag[r]) * au[r]) : 0u);
        }
    }
    __syncthreads();

    // ---- down: latent rows n in 16-row blocks (wave, wave + WAVES, ...), K = this slice's FS columns
    if (nmine > 0) {  // a wave beyond the row blocks (L < 16 * WAVES) has none
        uint4 hb[FS / 32];
#pragma unroll
        for (int s = 0; s < FS / 32; ++s) hb[s] = *reinterpret_cast<const uint4*>(Hs + j * HP + step_k<SPL>(s, kq));
        const int drow = j < nrows ? d.seg.dest_of(tl.seg, tl.row0 + j) : -1;
        float* out = drow >= 0 ? d.P + ((size_t)drow * d.nslices + slice) * L + 4 * kq : nullptr;
        auto compute = [&](const typename ER::WRaw (&w)[RB][KG], int b0) {
#pragma unroll
            for (int i = 0; i < RB; ++i) {
                if (b0 + i < nmine) {
                    f32x4 acc = f32x4{};
#pragma unroll
                    for (int g = 0; g < KG; ++g)
#pragma unroll
                        for (int t = 0; t < SPL; ++t)
                            acc = mfma16(ER::template frag<MXR>(w[i][g], t), hb[g * SPL + t], acc);
                    if (out) {
                        const int blk = wave + WAVES * (b0 + i);
                        *reinterpret_cast<float4*>(out + blk * 16) = make_float4(acc[0], acc[1], acc[2], acc[3]);
                    }
                }
            }
        };
        for (int b = 0; b < nmine; b += 2 * RB) {
            load_dn(wb, b + RB);
            compute(wa, b);
            load_dn(wa, b + 2 * RB);
            if (b + RB < nmine) compute(wb, b + RB);
        }
    }
    __syncthreads();  // Hs and red are rewritten by the next item
}

// A persistent grid walks the items (tile, slice); items past the segment's width are skipped.
template <int WAVES, int KSU, int CH, bool MX>
__global__ __launch_bounds__(64 * WAVES) void decode_experts_kernel(const DecodeExperts<MX> d) {
    using DS = DecodeShape<WAVES, KSU>;
    __shared__ __align__(16) uint16_t Hs[16 * DS::kHP];
    __shared__ float red[DS::kRed];
    const int nitems = *d.seg.ntiles * d.nslices;
    for (int item = blockIdx.x; item < nitems; item += gridDim.x) {
        const int tile = item / d.nslices, slice = item - tile * d.nslices;
        const Tile tl = d.seg.tiles[tile];
        typename ExpertRows<MX>::Mat mats[3];
        int Fseg;
        bool mx;
        segment_mats<MX>(d.experts, d.rec_bytes, d.shared, tl.seg, d.seg.E, d.F, d.Fs, d.L, mats, Fseg, mx);
        if (slice * DS::kFS >= Fseg) continue;
        if (mx)
            decode_item<WAVES, KSU, CH, MX, MX>(d, tl, slice, mats, Fseg, Hs, red);
        else
            decode_item<WAVES, KSU, CH, false, MX>(d, tl, slice, mats, Fseg, Hs, red);
    }
}

// m[t] = sum_q P[shared t][q] + sum_s w[t][s] * sum_q P[t k + s][q]   (bf16 out; q over the
// slices a segment has: ns_routed = F / FS, ns_shared = Fs / FS).  A block covers 256 latent
// columns of one token: thread (x, y) sums the slices of rows y, y + 8, ... for columns 4x..4x+3,
// then the rows are combined in fixed order (shared row first, then slots 0..k-1).
constexpr int kMergeRows = 8;

__global__ __launch_bounds__(64 * kMergeRows) void merge_slices_kernel(const float* __restrict__ P,
                                                                       const float* __restrict__ w, int T, int k,
                                                                       int L, int nslices, int ns_routed,
                                                                       int ns_shared, uint16_t* __restrict__ m16) {
    __shared__ float4 part[17][64];  // rows: slot s at s, the shared row at k (k <= 16)
    const int t = blockIdx.y;
    const int x = threadIdx.x & 63, yrow = threadIdx.x >> 6;
    const int c = blockIdx.x * 256 + 4 * x;
    const bool ok = c < L;
    const int nrow = k + (ns_shared > 0 ? 1 : 0);
    const size_t rs = (size_t)nslices * L;
    for (int r = yrow; r < nrow; r += kMergeRows) {
        const bool sh = r == k;
        const float* row = P + (sh ? (size_t)T * k + t : (size_t)t * k + r) * rs + c;
        const int nq = sh ? ns_shared : ns_routed;
        float4 y = make_float4(0.f, 0.f, 0.f, 0.f);
        if (ok) {
            // slices in batches of 8 loads in flight (clamped addresses), summed in slice order
            for (int q0 = 0; q0 < nq; q0 += 8) {
                float4 v[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) v[i] = *reinterpret_cast<const float4*>(row + (size_t)min(q0 + i, nq - 1) * L);
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    if (q0 + i < nq) {
                        y.x += v[i].x;
                        y.y += v[i].y;
                        y.z += v[i].z;
                        y.w += v[i].w;
                    }
            }
            if (!sh) {
                const float ws = w[(size_t)t * k + r];
                y = make_float4(ws * y.x, ws * y.y, ws * y.z, ws * y.w);
            }
        }
        part[r][x] = y;
    }
    __syncthreads();
    if (yrow == 0 && ok) {
        float4 acc = nrow > k ? part[k][x] : make_float4(0.f, 0.f, 0.f, 0.f);
        for (int s = 0; s < k; ++s) {
            const float4 v = part[s][x];
            acc.x += v.x;
            acc.y += v.y;
            acc.z += v.z;
            acc.w += v.w;
        }
        *reinterpret_cast<uint2*>(m16 + (size_t)t * L + c) = make_uint2(pack_bf2(acc.x, acc.y), pack_bf2(acc.z, acc.w));
    }
}

}  // namespace lmoe
