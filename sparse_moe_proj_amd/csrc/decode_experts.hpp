// Expert work of a small batch (decode / speculative verify, T <= 64 tokens) in two launches
// with no dependency between workgroups inside either launch.
//
// 1. Gate/up (decode_gu_kernel).  A work item is (tile, block): the tile's tokens (<= 16 rows of
//    one segment) and 16 consecutive columns f of the SwiGLU width; a wave computes the gate and
//    up rows of the block against the tokens (K = latent, weights streamed from HBM, double
//    buffered) and stores SiLU(g) * u into
//        H[segment row][f]
//    (bf16; fp16 for 4-bit segments, whose rows decode to fp16 MFMA operands).
//    Items are dealt evenly over the compute units, so every CU streams the same share.
// 2. Down and merge (decode_dc_kernel).  A workgroup owns 16 latent rows and one group of the
//    work list (the tiles are split into G contiguous groups).  Its waves take the group's tiles
//    in turn as one stream of weight chunks; for a tile, Y = H(tile rows) . down^T over the full
//    SwiGLU width (weights streamed, H rows read back from L2), and each row's result is added,
//    times its routing weight (1 for the shared expert), to the wave's per-token accumulator in
//    LDS.  The waves' accumulators are
//    then summed in wave order and written as the group's partial merged rows
//        mpart[g][t][latent]  (bf16).
//    The U projection sums the G partials (in group order) while staging its input.
//
// Every sum runs in a fixed order (tiles in work-list order within a wave, waves in order,
// groups in order), so results do not depend on scheduling.
#pragma once

#include "gemm_stream.hpp"
#include "problems.hpp"
#include "route.hpp"

namespace lmoe {

template <int Q>
struct DecodeExperts {
    SegSpace seg;
    const uint16_t* z16;   // [T][L]
    const uint16_t* z16h;  // [T][L] fp16 copy of z16, or null (4-bit rows then convert z16)
    const void* experts;
    size_t rec_bytes;
    const uint16_t* shared;
    int L, F, Fs, Hs;  // Hs = max(F, Fs): row pitch of H
    int nblocks;       // 16-row blocks of the widest segment: ceil(Hs / 16)
    uint16_t* H;       // [T*k + T][Hs] bf16, segment-row order
    const float* w;    // [T][k] routing weights (slot order)
    uint16_t* mpart;   // [G][T][zp] bf16 (zp = seg.zp: the latent width times the expert groups)
    int groups;        // G
    const int2* rowinfo;  // [T*k] (token, weight bits) of the routed row at each position
    int max_tiles;        // work-list capacity (entries past *seg.ntiles are not used)
};

// Row readers: R = ExpertRows<0> (bf16 rows, also the shared expert of a 4-bit layer) or
// Fp4Rows<Q> (4-bit rows).  The bf16 view of a 4-bit layer's (bf16) shared-expert matrices.
template <int Q>
__device__ __forceinline__ void bf16_mats(const typename ExpertRows<Q>::Mat (&m)[3], ExpertRows<0>::Mat (&b)[3]) {
#pragma unroll
    for (int i = 0; i < 3; ++i) b[i] = ExpertRows<0>::Mat{reinterpret_cast<const uint16_t*>(m[i].p), 1.f};
}

// ---- gate/up ----------------------------------------------------------------------------------
// tok: the token of this lane's segment row (row0 + min(j, nrows - 1)).
template <int CH, class R, class DE>
__device__ __forceinline__ void gu_item(const DE& d, const Tile& tl, int f0, const typename R::Mat (&mats)[3],
                                        int tok) {
    using ER = R;
    constexpr bool MXR = true;  // (the readers ignore it)
    constexpr int SPL = ER::kSPL;
    const int lane = threadIdx.x & 63;
    const int kq = lane >> 4;
    const int j = lane & 15;
    const int L = d.L;
    const int nrows = tl.nrows;
    const typename ER::Row rg = ER::row(mats[0], f0 + j, L), ru = ER::row(mats[1], f0 + j, L);
    // fp16 operands: the token row from the fp16 copy when there is one, else converted
    const bool xh = ER::kF16 && d.z16h != nullptr;
    const uint16_t* xr = (xh ? d.z16h : d.z16) + d.seg.z_off(tl.seg, tok, L);
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
                    if constexpr (ER::kF16) {
                        const uint4 xv = sel4(xok, xh ? x[i * SPL + t] : bf16x8_to_f16x8(x[i * SPL + t]));
                        ag = mfma16_f16(ER::template frag<MXR>(g[i], t), xv, ag);
                        au = mfma16_f16(ER::template frag<MXR>(u[i], t), xv, au);
                    } else {
                        const uint4 xv = sel4(xok, x[i * SPL + t]);
                        ag = mfma16(ER::template frag<MXR>(g[i], t), xv, ag);
                        au = mfma16(ER::template frag<MXR>(u[i], t), xv, au);
                    }
                }
    };
    load(ga, ua, xa, 0);
    for (int c = 0; c < nch; c += 2) {
        load(gbuf, ubuf, xb, c + 1);
        compute(ga, ua, xa, c);
        load(ga, ua, xa, c + 2);
        if (c + 1 < nch) compute(gbuf, ubuf, xb, c + 1);
    }
    // this lane holds f rows f0 + 4 kq + r (r = 0..3) of segment row j; H rows of 4-bit segments
    // are fp16 (the operand type of their down projection), else bf16
    if (xok) {
        const float tg = mats[0].ts, tu = mats[1].ts;  // tensor scales (NVFP4; else 1)
        float h[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) h[r] = silu(ag[r] * tg) * (au[r] * tu);
        const uint2 v = ER::kF16 ? make_uint2(pack_f16x2(h[0], h[1]), pack_f16x2(h[2], h[3]))
                                 : make_uint2(pack_bf2(h[0], h[1]), pack_bf2(h[2], h[3]));
        *reinterpret_cast<uint2*>(d.H + (size_t)(tl.row0 + j) * d.Hs + f0 + 4 * kq) = v;
    }
}

// Routing inputs of a gate/up launch that routes the batch itself (small T): every workgroup
// runs route_block on the logits into LDS (identical results in all of them), and workgroup 0
// also writes the routing outputs that later launches and the caller read.
struct GuRoute {
    const float* logits;   // [T][E] (hi half with a folded router)
    const float* logits2;  // [T][E] lo half, or null
    int BM, has_shared;
    RouteOut out;
};

// Gate/up work items are (tile, 16-row block of the SwiGLU width), in work-list order with the
// blocks of a tile adjacent.  The grid holds one workgroup per compute unit (W waves, at most
// one such workgroup fits a CU) and item i goes to workgroup i % grid, wave (i / grid) % W, so
// every CU streams the same number of items; blocks past the segment's width are skipped.
// RNV > 0: the launch routes the batch first (route_block with RNV logits per lane; dynamic LDS
// holds the work list, max_tiles entries); RNV = 0: the work list comes from global memory.
// CH: weight groups per load chunk of bf16 rows (32 values each); CH4: of 4-bit rows (128 values).
template <int W, int CH, int CH4, int Q, int RNV>
__global__ __launch_bounds__(64 * W) void decode_gu_kernel(const DecodeExperts<Q> d, const GuRoute r) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int j = lane & 15;
    const int T = d.seg.T, k = d.seg.k;
    extern __shared__ int4 gdsm[];
    __shared__ typename std::conditional<(RNV > 0), RouteScratch, int>::type sm;
    __shared__ int sntiles;
    Tile* stiles = reinterpret_cast<Tile*>(gdsm);
    int nt;
    const Tile* tiles;
    if constexpr (RNV > 0) {
        RouteOut out{};
        if (blockIdx.x == 0) out = r.out;
        route_block<RNV>(r.logits, r.logits2, T, d.seg.E, k, r.BM, r.has_shared, out, sm, stiles, &sntiles);
        __syncthreads();
        nt = sntiles;
        tiles = stiles;
    } else {
        nt = *d.seg.ntiles;
        tiles = d.seg.tiles;
    }
    const int nitems = nt * d.nblocks;
    for (int item = blockIdx.x + gridDim.x * wave; item < nitems; item += gridDim.x * W) {
        const int tile = item / d.nblocks, blk = item - tile * d.nblocks;
        const Tile tl = tiles[tile];
        typename ExpertRows<Q>::Mat mats[3];
        int Fseg;
        bool mx;
        segment_mats<Q>(d.experts, d.rec_bytes, d.shared, tl.seg, d.seg.E, d.F, d.Fs, d.L, mats, Fseg, mx);
        const int f0 = blk * 16;
        if (f0 >= Fseg) continue;  // widths are multiples of 16
        const int p = tl.row0 + min(j, tl.nrows - 1);
        int tok;
        if constexpr (RNV > 0)
            tok = tl.seg == d.seg.E ? p - T * k : sm.stok[p];
        else
            tok = d.seg.token_of(tl.seg, p);
        if constexpr (Q == 0) {
            gu_item<CH, ExpertRows<0>>(d, tl, f0, mats, tok);
        } else if (mx) {
            gu_item<CH4, Fp4Rows<Q>>(d, tl, f0, mats, tok);
        } else {
            ExpertRows<0>::Mat b[3];
            bf16_mats<Q>(mats, b);
            gu_item<CH, ExpertRows<0>>(d, tl, f0, b, tok);
        }
    }
}

// ---- gate/up with K split over the waves ----------------------------------------------------
// The same items in another arrangement: item i goes to workgroup i % grid, and all W waves of
// the workgroup work on it, wave w taking the contiguous run [G w / W, G (w + 1) / W) of the G
// weight groups along K (the latent dimension), at most MG groups.  Each wave's partial gate and
// up products (16 f rows x 16 segment rows) go to LDS; after one barrier per item, 256 threads
// sum them in wave order and store SiLU(g) * u.  The next item's weights and token rows are
// requested before the current item's products are reduced (two register sets), so every wave
// keeps its share of the weight stream in flight from item to item, and the per-item ALU work
// (4-bit decode, MFMA) is spread over all four SIMDs.
template <int W>
struct GuRed { float v[2][W][2][16 * 17]; };  // [buffer][wave][gate, up][f row * 17 + segment row]

// Items [first, end) of the workgroup's sequence (first, first + grid, ...) whose rows R reads.
template <int W, int MG, class R, int Q, class ItemOf>
__device__ __forceinline__ void gu_split_run(const DecodeExperts<Q>& d, int first, int end, ItemOf item_of,
                                             GuRed<W>& red, int& buf) {
    constexpr int SPL = R::kSPL;
    typedef typename R::WRaw WR;
    typedef decltype(item_of(0)) Ctx;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int kq = lane >> 4, j = lane & 15;
    const int G = d.L / (32 * SPL);
    const int ga = G * wave / W, gb = G * (wave + 1) / W;
    const int grid = gridDim.x;
    // the next item at or after m that has rows in its segment (the same for every wave)
    auto next_valid = [&](int m, Ctx& c) {
        for (; m < end; m += grid) {
            c = item_of(m);
            if (c.valid) return m;
        }
        return end;
    };
    // every call issues the same loads (clamped to a valid group), so the waits stay exact
    auto load = [&](WR (&w)[MG][2], uint4 (&x)[MG * SPL], const Ctx& c) {
#pragma unroll
        for (int i = 0; i < MG; ++i) {
            const int gi = max(min(ga + i, gb - 1), 0);
            w[i][0] = R::template load<true>(c.rg, gi, kq);
            w[i][1] = R::template load<true>(c.ru, gi, kq);
#pragma unroll
            for (int t = 0; t < SPL; ++t) x[i * SPL + t] = ld16(c.xr + step_k<SPL>(gi * SPL + t, kq));
        }
    };
    auto finish = [&](const WR (&w)[MG][2], const uint4 (&x)[MG * SPL], const Ctx& c) {
        f32x4 ag = f32x4{}, au = f32x4{};
        const bool xok = j < c.nrows;
#pragma unroll
        for (int i = 0; i < MG; ++i)
            if (ga + i < gb)
#pragma unroll
                for (int t = 0; t < SPL; ++t) {
                    if constexpr (R::kF16) {
                        const uint4 xv = sel4(xok, c.xh ? x[i * SPL + t] : bf16x8_to_f16x8(x[i * SPL + t]));
                        ag = mfma16_f16(R::template frag<true>(w[i][0], t), xv, ag);
                        au = mfma16_f16(R::template frag<true>(w[i][1], t), xv, au);
                    } else {
                        const uint4 xv = sel4(xok, x[i * SPL + t]);
                        ag = mfma16(R::template frag<true>(w[i][0], t), xv, ag);
                        au = mfma16(R::template frag<true>(w[i][1], t), xv, au);
                    }
                }
        // lane (kq, j) holds f rows 4 kq + r of segment row j
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            red.v[buf][wave][0][(4 * kq + r) * 17 + j] = ag[r];
            red.v[buf][wave][1][(4 * kq + r) * 17 + j] = au[r];
        }
        __syncthreads();
        // thread e: segment row e / 16, f row e % 16 (16 consecutive outputs of a row)
        if (threadIdx.x < 256) {
            const int sr = threadIdx.x >> 4, fr = threadIdx.x & 15;
            if (sr < c.nrows) {
                float g = 0.f, u = 0.f;
#pragma unroll
                for (int v = 0; v < W; ++v) {
                    g += red.v[buf][v][0][fr * 17 + sr];
                    u += red.v[buf][v][1][fr * 17 + sr];
                }
                const float h = silu(g * c.tg) * (u * c.tu);
                d.H[(size_t)(c.row0 + sr) * d.Hs + c.f0 + fr] =
                    R::kF16 ? __builtin_bit_cast(uint16_t, f16_sat(h)) : (uint16_t)f2bf(h);
            }
        }
        buf ^= 1;
    };
    Ctx cur, nxt;
    int m = next_valid(first, cur);
    if (m >= end) return;
    WR wa[MG][2], wb[MG][2];
    uint4 xa[MG * SPL], xb[MG * SPL];
    load(wa, xa, cur);
    while (true) {
        int mn = next_valid(m + grid, nxt);
        if (mn < end) load(wb, xb, nxt);
        finish(wa, xa, cur);
        if (mn >= end) return;
        cur = nxt;
        m = mn;
        mn = next_valid(m + grid, nxt);
        if (mn < end) load(wa, xa, nxt);
        finish(wb, xb, cur);
        if (mn >= end) return;
        cur = nxt;
        m = mn;
    }
}

// grid: one workgroup per compute unit; W waves.  RNV as for decode_gu_kernel.  MG: largest run
// of bf16 weight groups (32 values) a wave takes, MG4: of 4-bit groups (128 values).
template <int W, int MG, int MG4, int Q, int RNV>
__global__ __launch_bounds__(64 * W) void decode_gu_split_kernel(const DecodeExperts<Q> d, const GuRoute r) {
    const int j = threadIdx.x & 15;
    const int T = d.seg.T, k = d.seg.k, E = d.seg.E;
    extern __shared__ int4 gdsm[];
    __shared__ typename std::conditional<(RNV > 0), RouteScratch, int>::type sm;
    __shared__ int sntiles;
    __shared__ GuRed<W> red;
    Tile* stiles = reinterpret_cast<Tile*>(gdsm);
    int nt;
    const Tile* tiles;
    if constexpr (RNV > 0) {
        RouteOut out{};
        if (blockIdx.x == 0) out = r.out;
        route_block<RNV>(r.logits, r.logits2, T, E, k, r.BM, r.has_shared, out, sm, stiles, &sntiles);
        __syncthreads();
        nt = sntiles;
        tiles = stiles;
    } else {
        nt = *d.seg.ntiles;
        tiles = d.seg.tiles;
    }
    // items of tiles [0, nr) are routed, the rest (the shared expert's tiles, last in the list)
    // are not: in a 4-bit layer the two kinds are read through different row readers
    int nr = nt;
    if constexpr (Q != 0)
        while (nr > 0 && tiles[nr - 1].seg == E) --nr;
    auto item_of = [&](auto rtag, int item) {
        using R = typename decltype(rtag)::type;
        struct Ctx {
            typename R::Row rg, ru;
            const uint16_t* xr;
            int row0, nrows, f0;
            float tg, tu;
            bool valid, xh;
        };
        Ctx c;
        const int tile = item / d.nblocks, blk = item - tile * d.nblocks;
        const Tile tl = tiles[tile];
        typename ExpertRows<Q>::Mat mats[3];
        int Fseg;
        bool mx;
        segment_mats<Q>(d.experts, d.rec_bytes, d.shared, tl.seg, E, d.F, d.Fs, d.L, mats, Fseg, mx);
        c.f0 = blk * 16;
        c.valid = c.f0 < Fseg;  // widths are multiples of 16
        const int p = tl.row0 + min(j, tl.nrows - 1);
        int tok;
        if constexpr (RNV > 0)
            tok = tl.seg == E ? p - T * k : sm.stok[p];
        else
            tok = d.seg.token_of(tl.seg, p);
        if constexpr (std::is_same<R, ExpertRows<0>>::value) {
            ExpertRows<0>::Mat b[3];
            if constexpr (Q != 0)
                bf16_mats<Q>(mats, b);
            else
                for (int i = 0; i < 3; ++i) b[i] = mats[i];
            c.rg = R::row(b[0], c.f0 + j, d.L);
            c.ru = R::row(b[1], c.f0 + j, d.L);
        } else {
            c.rg = R::row(mats[0], c.f0 + j, d.L);
            c.ru = R::row(mats[1], c.f0 + j, d.L);
        }
        c.xh = R::kF16 && d.z16h != nullptr;
        c.xr = (c.xh ? d.z16h : d.z16) + d.seg.z_off(tl.seg, tok, d.L);
        c.row0 = tl.row0;
        c.nrows = tl.nrows;
        c.tg = mats[0].ts;
        c.tu = mats[1].ts;
        return c;
    };
    int buf = 0;
    const int nitems = nt * d.nblocks, nrouted = nr * d.nblocks;
    if constexpr (Q == 0) {
        auto of = [&](int item) { return item_of(TypeTag<ExpertRows<0>>{}, item); };
        gu_split_run<W, MG, ExpertRows<0>>(d, blockIdx.x, nitems, of, red, buf);
    } else {
        auto of4 = [&](int item) { return item_of(TypeTag<Fp4Rows<Q>>{}, item); };
        gu_split_run<W, MG4, Fp4Rows<Q>>(d, blockIdx.x, nrouted, of4, red, buf);
        // the workgroup's first shared item: the first of its sequence at or after nrouted
        const int g = gridDim.x;
        const int fs = nrouted + (int)(((unsigned)blockIdx.x + g - (unsigned)(nrouted % g)) % g);
        auto of16 = [&](int item) { return item_of(TypeTag<ExpertRows<0>>{}, item); };
        gu_split_run<W, MG, ExpertRows<0>>(d, fs, nitems, of16, red, buf);
    }
}

// ---- down + merge -----------------------------------------------------------------------------
// A wave's tiles i0, i0 + W, ... (positions [ib, ie) of its sequence) as one stream of chunks
// (CH weight groups of one tile each, read through R) with the next chunk always in flight,
// across tile boundaries too; each finished tile goes to `combine`.
template <int CH, class R, class Ctx, class CtxOf, class Combine>
__device__ __forceinline__ void dc_run(int ib, int ie, CtxOf ctx_of, Combine combine) {
    constexpr int SPL = R::kSPL;
    typedef typename R::WRaw WR;
    const int kq = (threadIdx.x & 63) >> 4;
    // every call issues the same number of loads (clamped groups), so the waits stay exact
    auto load = [&](WR (&w)[CH], uint4 (&h)[CH * SPL], const Ctx& c, int ch) {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int gi = min(ch * CH + i, c.groups - 1);
            w[i] = R::template load<true>(c.rw, gi, kq);
#pragma unroll
            for (int t = 0; t < SPL; ++t) h[i * SPL + t] = ld16(c.hr + step_k<SPL>(gi * SPL + t, kq));
        }
    };
    auto compute = [&](const WR (&w)[CH], const uint4 (&h)[CH * SPL], const Ctx& c, int ch, f32x4& acc) {
#pragma unroll
        for (int i = 0; i < CH; ++i)
            if (ch * CH + i < c.groups)
#pragma unroll
                for (int t = 0; t < SPL; ++t) {
                    if constexpr (R::kF16)
                        acc = mfma16_f16(R::template frag<true>(w[i], t), sel4(c.ok, h[i * SPL + t]), acc);
                    else
                        acc = mfma16(R::template frag<true>(w[i], t), sel4(c.ok, h[i * SPL + t]), acc);
                }
    };
    if (ib >= ie) return;
    Ctx cur = ctx_of(ib), nxt = cur;
    int i = ib, ch = 0;
    bool more = true;
    f32x4 acc = f32x4{};
    WR wa[CH], wb[CH];
    uint4 ha[CH * SPL], hb[CH * SPL];
    // buffers x hold chunk (cur, ch): request the chunk after it into y, then use x
    auto step = [&](WR (&wx)[CH], uint4 (&hx)[CH * SPL], WR (&wy)[CH], uint4 (&hy)[CH * SPL]) {
        const bool last = ch + 1 >= cur.nch;
        const bool next_tile = last && i + 1 < ie;
        if (next_tile) nxt = ctx_of(i + 1);
        // past the run's last chunk the request repeats the current one (never used)
        load(wy, hy, next_tile ? nxt : cur, next_tile ? 0 : (last ? ch : ch + 1));
        compute(wx, hx, cur, ch, acc);
        if (last) {
            combine(acc, cur);
            acc = f32x4{};
            if (next_tile) {
                cur = nxt;
                ++i;
                ch = 0;
            } else {
                more = false;
            }
        } else {
            ++ch;
        }
    };
    load(wa, ha, cur, 0);
    while (more) {
        step(wa, ha, wb, hb);
        if (!more) break;
        step(wb, hb, wa, ha);
    }
}

// grid (L / 16, G, expert groups); W waves; dynamic LDS: max_tiles Tiles, then T*k int2 row
// records, then max_tiles ints (with expert groups: the indices of the group's tiles).
// A wave's tiles stream as chunks with the next one always in flight (dc_run); in a 4-bit layer
// the routed tiles and the (bf16) shared-expert tiles, which come last in the work list, are two
// such runs.  The tile list and the rows' tokens and weights are copied to LDS once, so no chunk
// waits on a descriptor.  Every wave reaches the barriers (no early return).
template <int W, int CH, int CH4, int Q>
__global__ __launch_bounds__(64 * W) void decode_dc_kernel(const DecodeExperts<Q> d) {
    extern __shared__ int4 dsm[];
    __shared__ float macc[W][kDecodeMaxT][17];  // per wave: [token][latent row of the block] (+1 pad)
    __shared__ int sng;
    Tile* stiles = reinterpret_cast<Tile*>(dsm);
    int2* srow = reinterpret_cast<int2*>(dsm + d.max_tiles);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int kq = lane >> 4, j = lane & 15;
    const int n0 = blockIdx.x * 16, grp = blockIdx.y, xg = blockIdx.z;
    const int T = d.seg.T, k = d.seg.k, E = d.seg.E;
    int* sidx = reinterpret_cast<int*>(srow + T * k);
    const int ntall = *d.seg.ntiles;
    for (int i = threadIdx.x; i < d.max_tiles; i += 64 * W) stiles[i] = d.seg.tiles[i];
    for (int p = threadIdx.x; p < T * k; p += 64 * W) srow[p] = d.rowinfo[p];
    for (int i = lane; i < T * 17; i += 64) (&macc[wave][0][0])[i] = 0.f;
    __syncthreads();
    // with expert groups the workgroup takes only the tiles of its group xg (the shared expert is
    // in group 0): wave 0 lists them in work-list order
    const bool grouped = gridDim.z > 1;
    if (grouped) {
        if (wave == 0) {
            int cnt = 0;
            for (int base = 0; base < ntall; base += 64) {
                const int i = base + lane;
                bool in = false;
                if (i < ntall) {
                    const int sg = stiles[i].seg;
                    in = (sg == E ? 0 : sg / d.seg.Eg) == xg;
                }
                const uint64_t b = __ballot(in);
                if (in) sidx[cnt + __popcll(b & ((1ull << lane) - 1ull))] = i;
                cnt += __popcll(b);
            }
            if (lane == 0) sng = cnt;
        }
        __syncthreads();
    }
    const int nt = grouped ? sng : ntall;
    auto tile_at = [&](int i) -> const Tile& { return stiles[grouped ? sidx[i] : i]; };
    const int tb = (int)((long)grp * nt / d.groups), te = (int)((long)(grp + 1) * nt / d.groups);
    const int nmine = te - tb > wave ? (te - tb - wave + W - 1) / W : 0;

    // lane (kq, j): latent rows n0 + 4 kq + r of segment row j -> its token and weight
    auto combine = [&](const f32x4& acc, const auto& c) {
        if (!c.ok) return;
        const int p = c.row0 + j;
        int t;
        float wt;
        if (c.seg == E) {
            t = p - T * k;
            wt = 1.f;
        } else {
            const int2 ri = srow[p];
            t = ri.x;
            wt = __int_as_float(ri.y);
        }
        wt *= c.ts;
        if (t >= 0)
#pragma unroll
            for (int r = 0; r < 4; ++r) macc[wave][t][4 * kq + r] += wt * acc[r];
    };
    // tile context through row reader R (4-bit rows, or bf16 rows)
    auto make_ctx = [&](auto rtag, int i) {
        using R = typename decltype(rtag)::type;
        struct Ctx {
            typename R::Row rw;
            const uint16_t* hr;
            int groups, nch, row0, nrows, seg;
            bool ok;
            float ts;  // tensor scale of the down matrix (NVFP4; else 1)
        };
        const Tile tl = tile_at(tb + wave + i * W);
        typename ExpertRows<Q>::Mat mats[3];
        int Fseg;
        bool mx;
        segment_mats<Q>(d.experts, d.rec_bytes, d.shared, tl.seg, E, d.F, d.Fs, d.L, mats, Fseg, mx);
        Ctx c;
        typename R::Mat dm;
        if constexpr (std::is_same<R, ExpertRows<0>>::value) {
            dm = ExpertRows<0>::Mat{reinterpret_cast<const uint16_t*>(mats[2].p), 1.f};
        } else {
            dm = mats[2];
        }
        c.rw = R::row(dm, n0 + j, Fseg);
        c.hr = d.H + (size_t)(tl.row0 + min(j, tl.nrows - 1)) * d.Hs;
        c.groups = Fseg / (32 * R::kSPL);
        c.nch = (c.groups + (std::is_same<R, ExpertRows<0>>::value ? CH : CH4) - 1) /
                (std::is_same<R, ExpertRows<0>>::value ? CH : CH4);
        c.row0 = tl.row0;
        c.nrows = tl.nrows;
        c.seg = tl.seg;
        c.ok = j < tl.nrows;
        c.ts = mats[2].ts;
        return c;
    };
    if constexpr (Q == 0) {
        using R = ExpertRows<0>;
        auto ctx_of = [&](int i) { return make_ctx(TypeTag<R>{}, i); };
        dc_run<CH, R, decltype(ctx_of(0))>(0, nmine, ctx_of, combine);
    } else {
        // the wave's routed tiles come first, then its shared-expert tiles
        int ish = nmine;
        for (int i = 0; i < nmine; ++i)
            if (tile_at(tb + wave + i * W).seg == E) {
                ish = i;
                break;
            }
        auto ctx4 = [&](int i) { return make_ctx(TypeTag<Fp4Rows<Q>>{}, i); };
        dc_run<CH4, Fp4Rows<Q>, decltype(ctx4(0))>(0, ish, ctx4, combine);
        auto ctx16 = [&](int i) { return make_ctx(TypeTag<ExpertRows<0>>{}, i); };
        dc_run<CH, ExpertRows<0>, decltype(ctx16(0))>(ish, nmine, ctx16, combine);
    }
    __syncthreads();
    // thread e: token e / 16, latent row n0 + e % 16; the waves' sums in wave order
    for (int e = threadIdx.x; e < 16 * T; e += 64 * W) {
        const int t = e >> 4, r = e & 15;
        {
            float s = 0.f;
#pragma unroll
            for (int w = 0; w < W; ++w) s += macc[w][t][r];
            d.mpart[((size_t)grp * T + t) * d.seg.zp + (size_t)xg * d.L + n0 + r] = (uint16_t)f2bf(s);
        }
    }
}

}  // namespace lmoe
