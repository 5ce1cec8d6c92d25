// Routing of token batches: top-k selection with softmax weights (one wave per token) and the
// stable token -> expert permutation, as device functions shared by the routing launches and by
// the small-batch gate/up launch (which routes a batch of up to 64 tokens itself).
#pragma once

#include "common.hpp"
#include "launch.hpp"

namespace lmoe {

// Inclusive prefix sum over the wave by DPP: three shifts by 1, 2, 3 lanes of the inputs give
// each lane the sum of its quad-aligned window of 4, shifts by 4 and 8 lanes (upper banks of
// each row only) extend it to the row, and two row broadcasts (lane 15 into rows 1 and 3, lane
// 31 into rows 2 and 3) carry the rows' totals.  Lanes without a source add 0.
__device__ __forceinline__ int wave_incl_scan(int x) {
    int s = x;
    s += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);  // row_shr 1
    s += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);  // row_shr 2
    s += __builtin_amdgcn_update_dpp(0, x, 0x113, 0xF, 0xF, true);  // row_shr 3
    s += __builtin_amdgcn_update_dpp(0, s, 0x114, 0xF, 0xE, true);  // row_shr 4, banks 1-3
    s += __builtin_amdgcn_update_dpp(0, s, 0x118, 0xF, 0xC, true);  // row_shr 8, banks 2-3
    s += __builtin_amdgcn_update_dpp(0, s, 0x142, 0xA, 0xF, false);  // row_bcast 15, rows 1, 3
    s += __builtin_amdgcn_update_dpp(0, s, 0x143, 0xC, 0xF, false);  // row_bcast 31, rows 2, 3
    return s;
}

// Exclusive prefix sum over the block (one value per thread, blockDim a multiple of 64, at
// most 2048 threads).  tmp needs 33 ints of LDS.  Every thread must call it.
__device__ int block_excl_scan(int v, int* tmp, int* total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
    const int x = wave_incl_scan(v);
    __syncthreads();
    if (lane == 63) tmp[w] = x;
    __syncthreads();
    if (w == 0) {
        const int t = wave_incl_scan(lane < nw ? tmp[lane] : 0);
        if (lane < nw) tmp[lane] = t;
        if (lane == 63) tmp[32] = t;
    }
    __syncthreads();
    *total = tmp[32];
    return x - v + (w > 0 ? tmp[w - 1] : 0);
}

// ==============================================================================================
// top-k + softmax over the kept logits, one wave per token.  Lane l holds the logits of ids
// l, l+64, ... (NV per lane, E <= 64*NV) as order-preserving 32-bit keys.  Each lane sorts its
// keys in descending order with a stable network (adjacent swaps of strictly smaller keys only,
// so equal keys keep their ascending-id order); then k rounds take the wave-wide maximum of the
// lanes' first keys, the winner being the lowest id among equal maxima, and the winning lane
// drops its first key.  This is "larger value wins, lower id wins a tie".  The kept ids are
// written in ascending order with softmax weights over their logits.
// ==============================================================================================
__device__ __forceinline__ uint32_t order_key(float v) {
    const uint32_t u = __float_as_uint(v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t key) {
    return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

// Maximum over the wave, returned uniform: DPP within each row of 16 lanes (swap neighbours,
// swap pairs, rotate by 4, rotate by 8), then the two row broadcasts of wave_incl_scan (lane 15
// into rows 1 and 3, lane 31 into rows 2 and 3; other rows take max with 0), so lane 63 holds
// the maximum of all four rows and one scalar read returns it.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xF, 0xF, false));  // row_ror 4
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false));  // row_ror 8
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));  // row_bcast 15
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false));  // row_bcast 31
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Sum over the wave in a fixed order (same DPP tree as wave_max_u32), returned uniform.
__device__ __forceinline__ float wave_sum_f32(float v) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return (r0 + r1) + (r2 + r3);
}

// Top k of one token's logits (row of E <= 1024) by one wave.  Lanes 0 .. k-1 return a kept
// expert as (rank among the kept ids in ascending order) << 16 | id, with its softmax weight;
// other lanes return -1.
// row2 (optional): a second half of the logits, added to row (the folded router's lo half).
// The lane's logits (ids lane + 64 j) of a row and of its second half (without one, the row
// again, which wave_topk_select then ignores), as wave_topk_select takes them.  Only loads are
// issued (clamped addresses, no branch), so they are in flight together and nothing here waits
// for them.
template <int NV>
__device__ __forceinline__ void wave_topk_load(const float* __restrict__ row, const float* __restrict__ row2, int E,
                                               float (&v)[NV], float (&v2)[NV]) {
    const int lane = threadIdx.x & 63;
    const float* r2 = row2 ? row2 : row;
#pragma unroll
    for (int j = 0; j < NV; ++j) v[j] = row[min(lane + 64 * j, E - 1)];
#pragma unroll
    for (int j = 0; j < NV; ++j) v2[j] = r2[min(lane + 64 * j, E - 1)];
}

// The k rounds over the lanes' sorted runs: each round takes the wave-wide maximum of the lanes'
// first keys h[0] (the lowest id among equal maxima), lane r records it (key, id), and the winning
// lane drops its first key.  H keys per lane take part; returns false when some lane has won H
// times (its next key was not in the race, so the result may be wrong and the caller must run
// the rounds over the whole sorted run).
template <int H>
__device__ __forceinline__ bool wave_topk_rounds(uint32_t (&h)[H], int (&hid)[H], int k, bool check,
                                                 uint32_t& sel_key, int& sel_id) {
    const int lane = threadIdx.x & 63;
    int wins = 0;
    sel_key = 0;
    sel_id = -1;
#pragma unroll 1
    for (int r = 0; r < k; ++r) {
        const uint32_t m = wave_max_u32(h[0]);
        const uint64_t cand = __ballot(h[0] == m);
        int win = __ffsll((unsigned long long)cand) - 1;
        if (__popcll(cand) > 1) {  // equal maxima: the lowest id among the candidates
            const uint32_t lo = ~wave_max_u32(h[0] == m ? ~(uint32_t)hid[0] : 0u);
            win = __ffsll((unsigned long long)__ballot(h[0] == m && (uint32_t)hid[0] == lo)) - 1;
        }
        const int wid = __builtin_amdgcn_readlane(hid[0], win);
        if (lane == r) {
            sel_key = m;
            sel_id = wid;
        }
        if (lane == win) {
#pragma unroll
            for (int j = 0; j + 1 < H; ++j) {
                h[j] = h[j + 1];
                hid[j] = hid[j + 1];
            }
            h[H - 1] = 0u;
            ++wins;
        }
    }
    return !check || __ballot(wins >= H) == 0ull;
}

// Softmax over the kept logits (lanes 0 .. k-1 hold them in selection order) and each kept id's
// rank among the kept ids in ascending order.
__device__ __forceinline__ void wave_topk_finish(uint32_t sel_key, int sel_id, int k, int& out, float& out_w) {
    const int lane = threadIdx.x & 63;
    // the first winner holds the largest kept logit
    const float vmax = key_value((uint32_t)__builtin_amdgcn_readlane((int)sel_key, 0));
    const float e = lane < k ? expf(key_value(sel_key) - vmax) : 0.f;
    const float s = wave_sum_f32(e);
    // rank among the kept ids (distinct), ascending
    int pos = 0;
    for (int r = 0; r < k; ++r) pos += __builtin_amdgcn_readlane(sel_id, r) < sel_id ? 1 : 0;
    out = lane < k ? (pos << 16) | sel_id : -1;
    out_w = lane < k ? e / s : 0.f;
}

// Stable descending order of a lane's first P keys: P bubble passes from the end, each moving the
// largest remaining key to the front with strict comparisons (equal keys keep their order, i.e.
// ascending id).  P = N gives the whole run sorted.
template <int N, int P>
__device__ __forceinline__ void lane_sort_prefix(uint32_t (&key)[N], int (&id)[N]) {
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
        for (int j = N - 2; j >= p; --j) {
            const bool sw = key[j + 1] > key[j];
            const uint32_t ka = key[j], kb = key[j + 1];
            const int ia = id[j], ib = id[j + 1];
            key[j] = sw ? kb : ka;
            key[j + 1] = sw ? ka : kb;
            id[j] = sw ? ib : ia;
            id[j + 1] = sw ? ia : ib;
        }
}

template <int NV>
__device__ __forceinline__ void wave_topk_select(const float (&v1)[NV], const float (&v2)[NV], bool has2, int E, int k,
                                                 int& out, float& out_w) {
    const int lane = threadIdx.x & 63;
    uint32_t key[NV];
    int id[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const float v = has2 ? v1[j] + v2[j] : v1[j];
        // NaN counts as -inf (never ahead of a number); ids past E get key 0, below every value
        const float x = v == v ? v : -INFINITY;
        key[j] = lane + 64 * j < E ? order_key(x) : 0u;
        id[j] = lane + 64 * j;
    }
    uint32_t sel_key;
    int sel_id;
    // Most rounds take a lane's first few keys only: the first H keys of each lane race, which is
    // exact unless some lane wins H times; then the rounds run again over the whole sorted run.
    constexpr int H = NV < 4 ? NV : 4;
    if constexpr (H == NV) {
        lane_sort_prefix<NV, NV>(key, id);
        wave_topk_rounds<NV>(key, id, k, false, sel_key, sel_id);
    } else {
        uint32_t kf[NV];
        int idf[NV];
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            kf[j] = key[j];
            idf[j] = id[j];
        }
        lane_sort_prefix<NV, H>(key, id);
        uint32_t hk[H];
        int hi[H];
#pragma unroll
        for (int j = 0; j < H; ++j) {
            hk[j] = key[j];
            hi[j] = id[j];
        }
        if (!wave_topk_rounds<H>(hk, hi, k, true, sel_key, sel_id)) {
            lane_sort_prefix<NV, NV>(kf, idf);
            wave_topk_rounds<NV>(kf, idf, k, false, sel_key, sel_id);
        }
    }
    wave_topk_finish(sel_key, sel_id, k, out, out_w);
}

template <int NV>
__device__ __forceinline__ void wave_topk(const float* __restrict__ row, const float* __restrict__ row2, int E, int k,
                                          int& out, float& out_w) {
    float v[NV], v2[NV];
    wave_topk_load<NV>(row, row2, E, v, v2);
    wave_topk_select<NV>(v, v2, row2 != nullptr, E, k, out, out_w);
}

// ==============================================================================================
// Permutation.  Tokens are cut into blocks of 64; inside a block, bit tl of bm[2e + tl/32] marks
// that token tl chose expert e.  Because a token's ids are distinct, the stable rank of slot
// (t, s) inside expert e's segment is (slots of e in earlier blocks) + popcount of the bits of
// earlier tokens of the same block, so no sort is needed and the result is unique.
// ==============================================================================================
constexpr int kPermTB = 64;

__device__ __forceinline__ int bits_below(const uint32_t* bm, int e, int tl) {
    const uint32_t w0 = bm[2 * e], w1 = bm[2 * e + 1];
    return tl < 32 ? __popc(w0 & ((1u << tl) - 1u)) : __popc(w0) + __popc(w1 & ((1u << (tl - 32)) - 1u));
}

// rowinfo (optional, with the block's weights w): rowinfo[pos] = (token, weight bits) of the
// slot placed at pos.
__device__ void perm_scatter_block(const int32_t* __restrict__ ids, int T, int k, int E, int b, const uint32_t* bm,
                                   const int* seg_base /* per expert: first position for this block */,
                                   int32_t* __restrict__ perm, int32_t* __restrict__ inv, const float* w = nullptr,
                                   int2* __restrict__ rowinfo = nullptr) {
    const int t0 = b * kPermTB;
    const int nt = min(kPermTB, T - t0);
    for (int i = threadIdx.x; i < nt * k; i += blockDim.x) {
        const size_t f = (size_t)t0 * k + i;
        const int e = ids[f];
        if (e < 0 || e >= E) {
            inv[f] = -1;
            continue;
        }
        const int pos = seg_base[e] + bits_below(bm, e, i / k);
        perm[pos] = (int32_t)f;
        inv[f] = pos;
        if (rowinfo) rowinfo[pos] = make_int2(t0 + i / k, __float_as_int(w[i]));
    }
}

// LDS of route_block (E <= 1024, T <= 64, k <= 16).
struct RouteScratch {
    uint32_t bm[2 * 1024];  // per expert: bits of the tokens that chose it
    int soff[1024];         // per expert: segment start
    int tmp[33];
    int32_t sids[64 * 16];  // [T][k] chosen ids, ascending per token
    float sw[64 * 16];      // [T][k] their weights
    int stok[64 * 16];      // [T*k] token of the slot at each permuted position
};

// Routing and permutation of T <= 64 tokens by one workgroup (blockDim a multiple of 64, up to
// 1024; every thread must call it).  Each wave selects the experts of its tokens and marks them
// in the per-expert token bitmaps; one block scan of (count | tiles << 16) over the experts (each
// thread a contiguous run of them) gives the segment offsets and the work-list positions
// together (counts <= 1024 and tile counts <= 1024 never carry into each other); every slot is
// then placed at its stable rank (earlier tokens first) inside its expert's segment.  The work
// list (routed segments in expert order, each cut into <= BM-row tiles, then the shared
// segment) is also written to stiles / *sntiles when those are given.
template <int NV>
__device__ void route_block(const float* __restrict__ logits, const float* __restrict__ logits2, int T, int E, int k,
                            int BM, int has_shared, const RouteOut& g, RouteScratch& sm, Tile* stiles, int* sntiles) {
    const int nthr = blockDim.x, nwaves = nthr >> 6;
    const int tw = threadIdx.x >> 6;
    float v[NV], v2[NV];
    // the wave's first token's logits are requested before the bitmaps are cleared
    if (tw < T) wave_topk_load<NV>(logits + (size_t)tw * E, logits2 ? logits2 + (size_t)tw * E : nullptr, E, v, v2);
    for (int i = threadIdx.x; i < 2 * E; i += nthr) sm.bm[i] = 0;
    __syncthreads();
    for (int t = tw; t < T; t += nwaves) {
        int pid;
        float wt;
        if (t != tw) wave_topk_load<NV>(logits + (size_t)t * E, logits2 ? logits2 + (size_t)t * E : nullptr, E, v, v2);
        wave_topk_select<NV>(v, v2, logits2 != nullptr, E, k, pid, wt);
        if (pid >= 0) {
            const int pos = pid >> 16, e = pid & 0xffff;
            if (g.ids) g.ids[(size_t)t * k + pos] = e;
            if (g.w) g.w[(size_t)t * k + pos] = wt;
            sm.sids[t * k + pos] = e;
            sm.sw[t * k + pos] = wt;
            atomicOr(&sm.bm[2 * e + (t >> 5)], 1u << (t & 31));
        }
    }
    __syncthreads();
    // thread th owns experts [th * ept, th * ept + ept)
    const int ept = (E + nthr - 1) / nthr;
    const int e0 = threadIdx.x * ept;
    int run = 0;
    for (int i = 0; i < ept; ++i) {
        const int e = e0 + i;
        if (e < E) {
            const int cnt = __popc(sm.bm[2 * e]) + __popc(sm.bm[2 * e + 1]);
            run += cnt | (((cnt + BM - 1) / BM) << 16);
        }
    }
    int total;
    int packed = block_excl_scan(run, sm.tmp, &total);
    const int nslots = total & 0xffff, ntot = total >> 16;
    for (int i = 0; i < ept; ++i) {
        const int e = e0 + i;
        if (e >= E) break;
        const int cnt = __popc(sm.bm[2 * e]) + __popc(sm.bm[2 * e + 1]);
        const int nt = (cnt + BM - 1) / BM;
        const int off = packed & 0xffff, ts = packed >> 16;
        sm.soff[e] = off;
        if (g.offsets) g.offsets[e] = off;
        for (int j = 0; j < nt; ++j) {
            const Tile tl{e, off + j * BM, min(BM, cnt - j * BM), 0};
            if (g.tiles) g.tiles[ts + j] = tl;
            if (stiles) stiles[ts + j] = tl;
        }
        packed += cnt | (nt << 16);
    }
    if (threadIdx.x == 0 && g.offsets) g.offsets[E] = nslots;
    const int nsh = has_shared ? (T + BM - 1) / BM : 0;
    for (int j = threadIdx.x; j < nsh; j += nthr) {
        const Tile tl{E, T * k + j * BM, min(BM, T - j * BM), 0};
        if (g.tiles) g.tiles[ntot + j] = tl;
        if (stiles) stiles[ntot + j] = tl;
    }
    if (threadIdx.x == 0) {
        if (g.ntiles) *g.ntiles = ntot + nsh;
        if (sntiles) *sntiles = ntot + nsh;
    }
    for (int i = nslots + threadIdx.x; i < T * k; i += nthr) {
        if (g.perm) g.perm[i] = -1;
        if (g.rowinfo) g.rowinfo[i] = make_int2(-1, 0);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < T * k; i += nthr) {
        const int e = sm.sids[i];
        const int pos = sm.soff[e] + bits_below(sm.bm, e, i / k);
        sm.stok[pos] = i / k;
        if (g.perm) g.perm[pos] = i;
        if (g.inv) g.inv[i] = pos;
        if (g.rowinfo) g.rowinfo[pos] = make_int2(i / k, __float_as_int(sm.sw[i]));
    }
}

}  // namespace lmoe
