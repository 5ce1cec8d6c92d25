// Kernels of the latent-MoE block other than the MFMA GEMM templates, and the host-side
// launch wrappers for everything (no allocation, no synchronisation: enqueue only).
#include <hip/hip_ext.h>
#include <limits.h>

#include "decode_experts.hpp"
#include "experts_mx.hpp"
#include "gemm_stream.hpp"
#include "gemm_tile.hpp"
#include "launch.hpp"
#include "problems.hpp"
#include "route.hpp"
#include "small_proj.hpp"

namespace lmoe {

// ==============================================================================================
// block-wide helpers
// ==============================================================================================

// Sum over the block in a fixed order (wave butterflies, then wave 0..n-1).  red: 16 floats.
__device__ float block_sum(float v, float* red) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    __syncthreads();
    if (lane == 0) red[w] = v;
    __syncthreads();
    float s = 0.f;
    for (int i = 0; i < nw; ++i) s += red[i];
    return s;
}

// ==============================================================================================
// RMSNorm prologue: x16[t] = bf16(h[t] / sqrt(mean(h[t]^2) + eps))  (unit gain)
// ==============================================================================================
__global__ __launch_bounds__(256) void rmsnorm_bf16_kernel(const float* __restrict__ h, int H, float eps,
                                                           uint16_t* __restrict__ x16) {
    __shared__ float red[16];
    const float* row = h + (size_t)blockIdx.x * H;
    float s = 0.f;
    for (int i = threadIdx.x; i < H; i += blockDim.x) s += row[i] * row[i];
    const float tot = block_sum(s, red);
    const float r = 1.0f / sqrtf(tot / (float)H + eps);
    for (int i = threadIdx.x; i < H; i += blockDim.x) x16[(size_t)blockIdx.x * H + i] = (uint16_t)f2bf(row[i] * r);
}

template <int NV>
__device__ __forceinline__ void topk_token(const float* __restrict__ row, const float* __restrict__ row2, int E, int k,
                                           int32_t* __restrict__ ids, float* __restrict__ w) {
    int pid;
    float wt;
    wave_topk<NV>(row, row2, E, k, pid, wt);
    if (pid >= 0) {
        ids[pid >> 16] = pid & 0xffff;
        w[pid >> 16] = wt;
    }
}

// logits2 (optional): a second [T][E] half added to logits (the folded router's lo half)
template <int NV>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, const float* __restrict__ logits2,
                                                   int T, int E, int k, int32_t* __restrict__ ids, float* __restrict__ w) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    topk_token<NV>(logits + (size_t)t * E, logits2 ? logits2 + (size_t)t * E : nullptr, E, k, ids + (size_t)t * k,
                   w + (size_t)t * k);
}

__device__ void perm_bitmap(const int32_t* __restrict__ ids, int T, int k, int E, int b, uint32_t* bm) {
    const int t0 = b * kPermTB;
    const int nt = min(kPermTB, T - t0);
    for (int i = threadIdx.x; i < 2 * E; i += blockDim.x) bm[i] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < nt * k; i += blockDim.x) {
        const int e = ids[(size_t)t0 * k + i];
        if (e >= 0 && e < E) {
            const int tl = i / k;
            atomicOr(&bm[e * 2 + (tl >> 5)], 1u << (tl & 31));
        }
    }
    __syncthreads();
}

// Work list of <= BM-row tiles: routed segments in expert order, then the shared segment.  The
// calling thread holds experts e0 .. e0+N-1 (slot counts cnt), whose segments start at off and
// follow one another; every thread of the block must call it.
template <int N>
__device__ void write_tiles(const int (&cnt)[N], int off, int e0, int E, int T, int k, int BM, int has_shared,
                            Tile* tiles, int32_t* ntiles, int* tmp) {
    int nt = 0;
#pragma unroll
    for (int j = 0; j < N; ++j) nt += e0 + j < E ? (cnt[j] + BM - 1) / BM : 0;
    int ntot;
    int ts = block_excl_scan(nt, tmp, &ntot);
#pragma unroll
    for (int j = 0; j < N; ++j) {
        if (e0 + j >= E) break;
        for (int r = 0; r < cnt[j]; r += BM) tiles[ts++] = Tile{e0 + j, off + r, min(BM, cnt[j] - r), 0};
        off += cnt[j];
    }
    const int nsh = has_shared ? (T + BM - 1) / BM : 0;
    for (int j = threadIdx.x; j < nsh; j += blockDim.x) tiles[ntot + j] = Tile{E, T * k + j * BM, min(BM, T - j * BM), 0};
    if (threadIdx.x == 0) *ntiles = ntot + nsh;
}

// Whole permutation in one workgroup (T <= 64 tokens); every thread of the block must call it.
__device__ void perm_single_body(const int32_t* ids, int T, int k, int E, int32_t* __restrict__ offsets,
                                 int32_t* __restrict__ perm, int32_t* __restrict__ inv, int BM, Tile* tiles,
                                 int32_t* ntiles, int has_shared, uint32_t* bm, int* soff, int* tmp) {
    perm_bitmap(ids, T, k, E, 0, bm);
    const int e = threadIdx.x;
    const int cnt = e < E ? __popc(bm[2 * e]) + __popc(bm[2 * e + 1]) : 0;
    int total;
    const int off = block_excl_scan(cnt, tmp, &total);
    if (e < E) {
        offsets[e] = off;
        soff[e] = off;
    }
    if (e == 0) offsets[E] = total;
    for (int i = total + threadIdx.x; i < T * k; i += blockDim.x) perm[i] = -1;
    if (tiles) write_tiles<1>({cnt}, off, e, E, T, k, BM, has_shared, tiles, ntiles, tmp);
    __syncthreads();
    perm_scatter_block(ids, T, k, E, 0, bm, soff, perm, inv);
}

__global__ __launch_bounds__(1024) void perm_single_kernel(const int32_t* __restrict__ ids, int T, int k, int E,
                                                           int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
                                                           int32_t* __restrict__ inv, int BM, Tile* tiles,
                                                           int32_t* ntiles, int has_shared) {
    __shared__ uint32_t bm[2 * 1024];
    __shared__ int soff[1024];
    __shared__ int tmp[33];
    perm_single_body(ids, T, k, E, offsets, perm, inv, BM, tiles, ntiles, has_shared, bm, soff, tmp);
}

// Routing and permutation of a small batch (T <= 64) in one workgroup (route_block).
template <int NV>
__global__ __launch_bounds__(1024) void topk_perm_single_kernel(const float* __restrict__ logits,
                                                                const float* __restrict__ logits2, int T, int E, int k,
                                                                int32_t* __restrict__ ids, float* __restrict__ w,
                                                                int32_t* __restrict__ offsets,
                                                                int32_t* __restrict__ perm, int32_t* __restrict__ inv,
                                                                int BM, Tile* tiles, int32_t* ntiles, int has_shared,
                                                                int2* rowinfo) {
    __shared__ RouteScratch sm;
    route_block<NV>(logits, logits2, T, E, k, BM, has_shared, RouteOut{ids, w, offsets, perm, inv, tiles, ntiles, rowinfo},
                    sm, nullptr, nullptr);
}

__global__ __launch_bounds__(256) void perm_hist_kernel(const int32_t* __restrict__ ids, int T, int k, int E,
                                                        int32_t* __restrict__ hist) {
    __shared__ uint32_t bm[2 * 1024];
    perm_bitmap(ids, T, k, E, blockIdx.x, bm);
    for (int e = threadIdx.x; e < E; e += blockDim.x)
        hist[(size_t)blockIdx.x * E + e] = __popc(bm[2 * e]) + __popc(bm[2 * e + 1]);
}

// Per expert, the inclusive running count of its slots over the token blocks: incl[b][e] = sum of
// hist[0..b][e], so row nb-1 holds each expert's total.  Workgroup g takes experts [64g, 64g+64);
// its 16 waves split the blocks into 16 parts, each thread sums its part of one expert's column,
// the parts' sums meet in LDS, and each thread writes its part's running counts from the sum of
// the parts before it.
constexpr int kScanEPB = 64;
__global__ __launch_bounds__(1024) void perm_scan_kernel(const int32_t* __restrict__ hist, int nb, int E,
                                                         int32_t* __restrict__ incl) {
    constexpr int kP = 1024 / kScanEPB, kBatch = 16;
    __shared__ int psum[1024];  // [part][expert of the workgroup]
    const int el = threadIdx.x % kScanEPB, part = threadIdx.x / kScanEPB;
    const int e = blockIdx.x * kScanEPB + el;
    const bool act = e < E;
    const int b_lo = act ? (int)((long)nb * part / kP) : 0, b_hi = act ? (int)((long)nb * (part + 1) / kP) : 0;
    auto batch = [&](int b0, int (&h)[kBatch]) {
#pragma unroll
        for (int u = 0; u < kBatch; ++u) h[u] = hist[(size_t)min(b0 + u, b_hi - 1) * E + e];
    };
    int sum = 0;
    for (int b0 = b_lo; b0 < b_hi; b0 += kBatch) {
        int h[kBatch];
        batch(b0, h);
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
            if (b0 + u < b_hi) sum += h[u];
    }
    psum[threadIdx.x] = sum;
    __syncthreads();
    if (!act) return;
    int run = 0;
    for (int q = 0; q < part; ++q) run += psum[q * kScanEPB + el];
    for (int b0 = b_lo; b0 < b_hi; b0 += kBatch) {
        int h[kBatch];
        batch(b0, h);
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
            if (b0 + u < b_hi) {
                run += h[u];
                incl[(size_t)(b0 + u) * E + e] = run;
            }
    }
}

// Block b scatters the slots of its tokens.  Every block scans the experts' totals (the last row
// of incl, four experts a thread) into the segment offsets; block b's first position for expert e
// is offsets[e] + incl[b-1][e].  Block 0 also writes the offsets and the work list, and the blocks
// together mark the positions past the last routed slot (perm = -1).
__global__ __launch_bounds__(256) void perm_scatter_kernel(const int32_t* __restrict__ ids, int T, int k, int E, int nb,
                                                           const int32_t* __restrict__ incl,
                                                           int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
                                                           int32_t* __restrict__ inv, int BM, Tile* tiles,
                                                           int32_t* ntiles, int has_shared) {
    constexpr int kEPT = 1024 / 256;
    __shared__ uint32_t bm[2 * 1024];
    __shared__ int sbase[1024];
    __shared__ int tmp[33];
    // the totals and the previous block's running counts load while the bitmap is built
    const int32_t* tot = incl + (size_t)(nb - 1) * E;
    const int32_t* prev = incl + (size_t)max((int)blockIdx.x - 1, 0) * E;
    const int e0 = threadIdx.x * kEPT;
    int c[kEPT], pb[kEPT], s = 0;
#pragma unroll
    for (int j = 0; j < kEPT; ++j) {
        c[j] = e0 + j < E ? tot[e0 + j] : 0;
        pb[j] = e0 + j < E && blockIdx.x > 0 ? prev[e0 + j] : 0;
    }
    perm_bitmap(ids, T, k, E, blockIdx.x, bm);
#pragma unroll
    for (int j = 0; j < kEPT; ++j) s += c[j];
    int total;
    const int off0 = block_excl_scan(s, tmp, &total);
    int off = off0;
#pragma unroll
    for (int j = 0; j < kEPT; ++j) {
        if (e0 + j < E) {
            sbase[e0 + j] = off + pb[j];
            if (blockIdx.x == 0) offsets[e0 + j] = off;
        }
        off += c[j];
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) offsets[E] = total;
    for (int i = total + blockIdx.x * blockDim.x + threadIdx.x; i < T * k; i += gridDim.x * blockDim.x) perm[i] = -1;
    if (blockIdx.x == 0 && tiles) write_tiles<kEPT>(c, off0, e0, E, T, k, BM, has_shared, tiles, ntiles, tmp);
    __syncthreads();
    perm_scatter_block(ids, T, k, E, blockIdx.x, bm, sbase, perm, inv);
}

// ==============================================================================================
// combine: m[t] = Y[T*k + t] (shared, weight 1) + sum_s w[t][s] * Y[t*k + s], slots in order
// ==============================================================================================
// 8 consecutive values of Y as they are stored (BF16: bf16 path, bf16 out; else the fp32 path,
// fp32 out), and as fp32
template <bool BF16>
struct Y8 {
    typename std::conditional<BF16, uint4, float4>::type a, b;
};
// The rows are read once per step: non-temporal loads, so that they do not push the merged rows
// (read next by the U projection) out of the caches (16K tokens: combine 144 -> 110 us, U 158 ->
// 152 us against plain loads).
template <bool BF16>
__device__ __forceinline__ Y8<BF16> load_y8(const void* Y, size_t off) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    typedef float f32x4v __attribute__((ext_vector_type(4)));
    Y8<BF16> r;
    if constexpr (BF16) {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(Y) + off));
        r.a = make_uint4(v.x, v.y, v.z, v.w);
    } else {
        const f32x4v* p = reinterpret_cast<const f32x4v*>(static_cast<const float*>(Y) + off);
        const f32x4v v0 = __builtin_nontemporal_load(p), v1 = __builtin_nontemporal_load(p + 1);
        r.a = make_float4(v0.x, v0.y, v0.z, v0.w);
        r.b = make_float4(v1.x, v1.y, v1.z, v1.w);
    }
    return r;
}
template <bool BF16>
__device__ __forceinline__ void y8_f32(const Y8<BF16>& r, float (&v)[8]) {
    if constexpr (BF16) {
        const uint32_t u[4] = {r.a.x, r.a.y, r.a.z, r.a.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(u[i] << 16);
            v[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
        }
    } else {
        v[0] = r.a.x, v[1] = r.a.y, v[2] = r.a.z, v[3] = r.a.w;
        v[4] = r.b.x, v[5] = r.b.y, v[6] = r.b.z, v[7] = r.b.w;
    }
}

// grid (L / 2048, min(T, 65535), expert groups), tokens t = blockIdx.y, + gridDim.y, ...: group
// g's merged row m_g goes to columns g * L .. of m [T][groups * L]; a slot counts for group
// ids / Eg (ids null: one group), the shared expert for group 0.  A thread sums 8 columns: the
// shared row, then the slots in order (fp32); all of a token's rows are requested (16-byte
// loads) before the first is added, so their loads are in flight together.
template <bool OUT_BF16>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ Y, const float* __restrict__ w, int T,
                                                      int k, int L, int has_shared, void* __restrict__ m,
                                                      const int32_t* __restrict__ ids, int Eg) {
    constexpr int KM = 16;  // top_k <= 16
    const int g = blockIdx.z;
    const int c = (blockIdx.x * blockDim.x + threadIdx.x) * 8;
    if (c >= L) return;
    const size_t mp = (size_t)gridDim.z * L;
    for (int t = blockIdx.y; t < T; t += gridDim.y) {
        // every row of the token (shared expert, then the slots) is requested before any is used,
        // so a token costs one round trip; the sum keeps the order shared, slot 0, 1, ...
        const bool sh = has_shared && g == 0;
        Y8<OUT_BF16> rsh;
        if (sh) rsh = load_y8<OUT_BF16>(Y, ((size_t)T * k + t) * L + c);
        Y8<OUT_BF16> raw[KM];
        float ws[KM];
        bool use[KM];
#pragma unroll
        for (int s = 0; s < KM; ++s) {
            use[s] = s < k && (!ids || ids[(size_t)t * k + s] / Eg == g);
            ws[s] = use[s] ? w[(size_t)t * k + s] : 0.f;
            if (use[s]) raw[s] = load_y8<OUT_BF16>(Y, ((size_t)t * k + s) * L + c);
        }
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (sh) y8_f32<OUT_BF16>(rsh, acc);
#pragma unroll
        for (int s = 0; s < KM; ++s) {
            if (!use[s]) continue;
            float y[8];
            y8_f32<OUT_BF16>(raw[s], y);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += ws[s] * y[e];
        }
        if (OUT_BF16) {
            const uint4 o = make_uint4(pack_bf2(acc[0], acc[1]), pack_bf2(acc[2], acc[3]), pack_bf2(acc[4], acc[5]),
                                       pack_bf2(acc[6], acc[7]));
            *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(m) + t * mp + (size_t)g * L + c) = o;
        } else {
            float4* o = reinterpret_cast<float4*>(reinterpret_cast<float*>(m) + t * mp + (size_t)g * L + c);
            o[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
            o[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
        }
    }
}

// ==============================================================================================
// plain fp32 path (fp32 storage end to end): one thread per output element, sequential K.
// ==============================================================================================
// mode 0: out = x.W^T ; 2: out += x.W^T ; bias (router) optional
__global__ __launch_bounds__(256) void f32_proj_kernel(const float* __restrict__ x, const float* __restrict__ W,
                                                       const float* __restrict__ bias, int T, int N, int K, int mode,
                                                       float* __restrict__ out) {
    const int n = blockIdx.x * blockDim.x + threadIdx.x;
    if (n >= N) return;
    for (int t = blockIdx.y; t < T; t += gridDim.y) {
        const float* xr = x + (size_t)t * K;
        const float* wr = W + (size_t)n * K;
        float acc = 0.f;
        for (int i = 0; i < K; ++i) acc = fmaf(xr[i], wr[i], acc);
        if (bias) acc += bias[n];
        float* o = out + (size_t)t * N + n;
        if (mode == 2)
            *o += acc;
        else
            *o = acc;
    }
}

struct F32Seg {
    const float* z;
    const int32_t* ids;
    const int32_t* perm;
    const float* experts;
    const float* shared;
    int T, k, L, F, Fs, Hs;
    // resolve segment row p: token, width and the expert record; false if p is a dropped slot
    __device__ bool resolve(int p, int& token, int& Fseg, const float*& rec) const {
        if (p < T * k) {
            const int slot = perm[p];
            if (slot < 0) return false;
            token = slot / k;
            Fseg = F;
            rec = experts + (size_t)ids[slot] * 3 * F * L;
        } else {
            token = p - T * k;
            Fseg = Fs;
            rec = shared;
        }
        return true;
    }
};

__global__ __launch_bounds__(256) void f32_up_kernel(const F32Seg s, int R, float* __restrict__ H) {
    const int f = blockIdx.x * blockDim.x + threadIdx.x;
    for (int p = blockIdx.y; p < R; p += gridDim.y) {
        int token, Fseg;
        const float* g;
        if (!s.resolve(p, token, Fseg, g) || f >= Fseg) continue;
        const float* u = g + (size_t)Fseg * s.L;
        const float* zr = s.z + (size_t)token * s.L;
        float a = 0.f, b = 0.f;
        for (int i = 0; i < s.L; ++i) {
            a = fmaf(zr[i], g[(size_t)f * s.L + i], a);
            b = fmaf(zr[i], u[(size_t)f * s.L + i], b);
        }
        H[(size_t)p * s.Hs + f] = a / (1.0f + expf(-a)) * b;
    }
}

__global__ __launch_bounds__(256) void f32_down_kernel(const F32Seg s, int R, const float* __restrict__ H,
                                                       float* __restrict__ Y) {
    const int n = blockIdx.x * blockDim.x + threadIdx.x;
    if (n >= s.L) return;
    for (int p = blockIdx.y; p < R; p += gridDim.y) {
        int token, Fseg;
        const float* g;
        if (!s.resolve(p, token, Fseg, g)) continue;
        const float* d = g + 2 * (size_t)Fseg * s.L + (size_t)n * Fseg;
        const float* hr = H + (size_t)p * s.Hs;
        float acc = 0.f;
        for (int f = 0; f < Fseg; ++f) acc = fmaf(hr[f], d[f], acc);
        const int dest = p < s.T * s.k ? s.perm[p] : p;
        Y[(size_t)dest * s.L + n] = acc;
    }
}

// ==============================================================================================
// launch wrappers
// ==============================================================================================
namespace {
inline unsigned cdiv(long a, long b) { return (unsigned)((a + b - 1) / b); }
inline hipError_t last() { return hipGetLastError(); }

// Shapes of the weight-streaming kernels: waves per workgroup, K slices per 16-row block, and
// weight loads per matrix in one pipelined chunk.
#ifndef LMOE_PROJ_WAVES
#define LMOE_PROJ_WAVES 8
#endif
#ifndef LMOE_PROJ_KS
#define LMOE_PROJ_KS 8
#endif
#ifndef LMOE_UP_WAVES
#define LMOE_UP_WAVES 4
#endif
#ifndef LMOE_UP_KS
#define LMOE_UP_KS 1
#endif
#ifndef LMOE_DOWN_WAVES
#define LMOE_DOWN_WAVES 4
#endif
#ifndef LMOE_DOWN_KS
#define LMOE_DOWN_KS 1
#endif
#ifndef LMOE_CHUNK
#define LMOE_CHUNK 4
#endif
#ifndef LMOE_PROJ_CHUNK
#define LMOE_PROJ_CHUNK 1
#endif
#ifndef LMOE_GU_WAVES
#define LMOE_GU_WAVES 8
#endif
#ifndef LMOE_GU_CHUNK
#define LMOE_GU_CHUNK 4
#endif
#ifndef LMOE_GU_SPLIT
#define LMOE_GU_SPLIT 1
#endif
#ifndef LMOE_GU_CHUNK4
#define LMOE_GU_CHUNK4 1
#endif
#ifndef LMOE_DC_CHUNK4
#define LMOE_DC_CHUNK4 2
#endif
#ifndef LMOE_DC_WAVES
#define LMOE_DC_WAVES 8
#endif
#ifndef LMOE_DC_CHUNK
#define LMOE_DC_CHUNK 4
#endif
#ifndef LMOE_DC_GROUPS
#define LMOE_DC_GROUPS 2
#endif
#ifndef LMOE_SP_WAVES
#define LMOE_SP_WAVES 8
#endif
#ifndef LMOE_SP_SMAX
#define LMOE_SP_SMAX 10
#endif
#ifndef LMOE_TILE_M
#define LMOE_TILE_M 128
#endif
#ifndef LMOE_TILE_N
#define LMOE_TILE_N 128
#endif
#ifndef LMOE_PIPE_M
#define LMOE_PIPE_M 128
#endif
#ifndef LMOE_PIPE_N
#define LMOE_PIPE_N 256
#endif
#ifndef LMOE_PIPE_NS
#define LMOE_PIPE_NS 3
#endif
#ifndef LMOE_PIPE_WR  // wave grid of a pipelined GEMM workgroup (rows x columns of wave tiles)
#define LMOE_PIPE_WR 2
#endif
#ifndef LMOE_PIPE_WC
#define LMOE_PIPE_WC 4
#endif
#ifndef LMOE_PIPE_PROJ
#define LMOE_PIPE_PROJ 1
#endif
#ifndef LMOE_PIPE_PERSIST
#define LMOE_PIPE_PERSIST 1
#endif
#ifndef LMOE_STREAM_GRID
#define LMOE_STREAM_GRID 2048
#endif
constexpr int kPW = LMOE_PROJ_WAVES, kPKS = LMOE_PROJ_KS;
constexpr int kUW = LMOE_UP_WAVES, kUKS = LMOE_UP_KS;
constexpr int kDW = LMOE_DOWN_WAVES, kDKS = LMOE_DOWN_KS;
constexpr int kChunk = LMOE_CHUNK;
constexpr int kProjChunk = LMOE_PROJ_CHUNK;
// Tile shape of the many-token GEMMs (projections, router, experts): 4 waves of (M/2) x (N/2).
using TileL = TileShape<LMOE_TILE_M, LMOE_TILE_N, 2, 2>;
// Pipelined (global -> LDS copies, LMOE_PIPE_NS stages) GEMM for the experts (and, with
// LMOE_PIPE_PROJ, the projections).
#ifndef LMOE_PIPE
#define LMOE_PIPE 1
#endif
using PipeL = PipeShape<LMOE_PIPE_M, LMOE_PIPE_N, LMOE_PIPE_NS, LMOE_PIPE_WR, LMOE_PIPE_WC>;
// The dense projections of large batches (D, U): every tile is full (no segments), so they may
// take a taller tile than the experts' work list allows.
#ifndef LMOE_PROJ_PIPE_M
#define LMOE_PROJ_PIPE_M LMOE_PIPE_M
#endif
#ifndef LMOE_PROJ_PIPE_N
#define LMOE_PROJ_PIPE_N LMOE_PIPE_N
#endif
#ifndef LMOE_PROJ_PIPE_NS
#define LMOE_PROJ_PIPE_NS LMOE_PIPE_NS
#endif
#ifndef LMOE_PROJ_PIPE_WR
#define LMOE_PROJ_PIPE_WR LMOE_PIPE_WR
#endif
#ifndef LMOE_PROJ_PIPE_WC
#define LMOE_PROJ_PIPE_WC LMOE_PIPE_WC
#endif
using PipeP = PipeShape<LMOE_PROJ_PIPE_M, LMOE_PROJ_PIPE_N, LMOE_PROJ_PIPE_NS, LMOE_PROJ_PIPE_WR, LMOE_PROJ_PIPE_WC>;
// Big tiles of the large-batch bf16 expert GEMMs: 256 x 256 with 8 waves of 128 x 64, two stages
// (128 KB of LDS).  A 128 x 256 tile moves 48 KB from L2 into LDS per 64-column stage for 4.2
// MFLOP, about 100 GB/s per CU at the matrix cores' rate; the 256 x 256 tile halves the bytes per
// flop.  Segments take whole big tiles and put their last rows in a 128-row tile when at most 128
// are left (so the padding stays that of 128-row tiles).
#ifndef LMOE_BIG_TILES
#define LMOE_BIG_TILES 1
#endif
#ifndef LMOE_BIG_WR
#define LMOE_BIG_WR 2
#endif
#ifndef LMOE_BIG_WC
#define LMOE_BIG_WC 4
#endif
#ifndef LMOE_BIG_BK
#define LMOE_BIG_BK 64
#endif
#ifndef LMOE_BIG_NS
#define LMOE_BIG_NS 2
#endif
using PipeB = PipeShape<256, LMOE_PIPE_N, LMOE_BIG_NS, LMOE_BIG_WR, LMOE_BIG_WC, LMOE_BIG_BK>;
// cost of a round of 256-row tiles over the CUs, in hundredths of a round of 128-row tiles
// (measured at 16384 x 1792 x 2560: 102 against 61 us per round; at 160 the U projection of
// 16384 tokens, 3 rounds against 5, takes the 256-row tiles: 160 against 167 us)
#ifndef LMOE_BIG_ROUND_COST
#define LMOE_BIG_ROUND_COST 160
#endif
constexpr long kBigRoundCost = LMOE_BIG_ROUND_COST;
static_assert(PipeB::kBN == PipeL::kBN, "big and small tiles cover the same columns per tile");

// Persistent launch: at most LMOE_STREAM_GRID workgroups walk max_tiles x row-group items.
template <int W, int KS, int NMAT, class P, int CH0 = kChunk>
hipError_t launch_stream(const P& p, int max_tiles, int nrows_max, hipStream_t s) {
    constexpr int CH = P::kSPL == 1 ? CH0 : 1;
    const int rgroups = (int)cdiv(nrows_max, 16 * (W / KS));
    const long items = (long)max_tiles * rgroups;
    const dim3 grid((unsigned)std::min<long>(items, LMOE_STREAM_GRID)), block(64 * W);
    hipLaunchKernelGGL((stream_gemm_kernel<W, KS, NMAT, CH, P>), grid, block, 0, s, p, rgroups);
    return last();
}
}  // namespace

// Compute units of the current device (cached per device).
int cu_count() {
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cache[dev]) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
        cache[dev] = cus;
    }
    return cache[dev];
}

// Workgroups of `kernel` that fit on the current device at once (cached per kernel and device).
template <class K>
int resident_blocks(K kernel, int threads) {
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cache[dev]) {
        int per_cu = 0, cus = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess || per_cu < 1)
            per_cu = 1;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 1;
        cache[dev] = per_cu * cus;
    }
    return cache[dev];
}

hipError_t launch_rmsnorm(const float* h, int T, int H, uint16_t* x16, hipStream_t s) {
    hipLaunchKernelGGL(rmsnorm_bf16_kernel, dim3(T), dim3(256), 0, s, h, H, 1e-6f, x16);
    return last();
}

// Lets a small-batch projection kernel take up to kSmallProjLds bytes of dynamic LDS (once per kernel).
template <int XM>
hipError_t small_proj_launch(const SmallProj& p, hipStream_t s) {
    auto k = small_proj_kernel<LMOE_SP_WAVES, LMOE_SP_SMAX, XM>;
    static const hipError_t attr =
        hipFuncSetAttribute(reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize, (int)kSmallProjLds);
    if (attr != hipSuccess) return attr;
    // one workgroup per row block up to one per CU; beyond that the workgroups take several
    // (a multiple of KG: workgroup w takes K group w % KG)
    const long grid = std::max<long>(std::min<long>(cdiv(p.N, 16) * p.KG, cu_count()) / p.KG * p.KG, p.KG);
    hipLaunchKernelGGL(k, dim3((unsigned)grid), dim3(64 * LMOE_SP_WAVES), small_proj_lds(p.K), s, p);
    return last();
}

#ifndef LMOE_ROWS_PROJ
#define LMOE_ROWS_PROJ 1
#endif
// Whether rows_proj_kernel takes a small-batch projection of reduction width K (its K range per
// wave fits the registers) with G partial inputs (XM 1).
bool rows_proj_fits(int T, int K, int XM, int G = 1) {
    return LMOE_ROWS_PROJ && T <= 16 * kSmallProjGroups && K % 32 == 0 &&
           (K / 32 + LMOE_SP_WAVES - 1) / LMOE_SP_WAVES <= rows_proj_smax(XM) && G <= kRowsMaxG;
}

// rows_proj_kernel over R = N (+ 2E router rows) rows: an even share of consecutive rows per CU.
template <int XM>
hipError_t rows_proj_launch(RowsProj p, hipStream_t s) {
    const long R = (long)p.N + (p.Gr ? 2L * p.E : 0);
    p.rpw = (int)cdiv(R, cu_count());
    p.eps = 1e-6f;
    hipLaunchKernelGGL((rows_proj_kernel<LMOE_SP_WAVES, XM>), dim3(cdiv(R, p.rpw)), dim3(64 * LMOE_SP_WAVES), 0, s, p);
    return last();
}

hipError_t launch_proj_router_bf16(const uint16_t* x, const uint16_t* D, const uint16_t* Gr, const float* br, int T,
                                  int L, int H, int E, float* z32, uint16_t* z16, float* logits, hipStream_t s,
                                  uint16_t* z16h, const float* hnorm) {
    if (rows_proj_fits(T, H, hnorm ? 2 : 0)) {
        const RowsProj p{x, hnorm, 0, D, T, L, H, 0, z32, z16, z16h, Gr, br, E, logits, 0, 0.f};
        return hnorm ? rows_proj_launch<2>(p, s) : rows_proj_launch<0>(p, s);
    }
    if (!small_proj_fits(T, H)) return hipErrorInvalidValue;
    SmallProj p{x, hnorm, 0, D, T, L, H, 0, z32, z16, Gr, br, E, logits, z16h};
    const dim3 grid((unsigned)std::min<long>(cdiv(L, 16) + 2 * cdiv(E, 16), cu_count()));
    if (hnorm) {
        auto k = small_proj_kernel<LMOE_SP_WAVES, LMOE_SP_SMAX, 2>;
        static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)kSmallProjLds);
        if (attr != hipSuccess) return attr;
        hipLaunchKernelGGL(k, grid, dim3(64 * LMOE_SP_WAVES), small_proj_lds(H), s, p);
    } else {
        auto k = small_proj_kernel<LMOE_SP_WAVES, LMOE_SP_SMAX, 0>;
        static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)kSmallProjLds);
        if (attr != hipSuccess) return attr;
        hipLaunchKernelGGL(k, grid, dim3(64 * LMOE_SP_WAVES), small_proj_lds(H), s, p);
    }
    return last();
}

// G = Wr . D in fp32 (ascending latent order), stored as hi = bf16(G), lo = bf16(G - hi):
// Gr [E][2][H].  One thread per (e, h); the block's 256 h share the Wr row.  With expert groups
// (Eg experts each) row e uses its group's D, rows (e / Eg) * L ...
__global__ __launch_bounds__(256) void fold_router_kernel(const uint16_t* __restrict__ D, const uint16_t* __restrict__ Wr,
                                                          int E, int L, int H, int Eg, uint16_t* __restrict__ Gr) {
    const int h = blockIdx.x * 256 + threadIdx.x, e = blockIdx.y;
    if (h >= H) return;
    const uint16_t* wr = Wr + (size_t)e * L;
    const uint16_t* dg = D + (size_t)(e / Eg) * L * H;
    float acc = 0.f;
    for (int l = 0; l < L; ++l) acc = fmaf(bf2f(wr[l]), bf2f(dg[(size_t)l * H + h]), acc);
    const uint32_t hi = f2bf(acc);
    Gr[(size_t)e * 2 * H + h] = (uint16_t)hi;
    Gr[(size_t)e * 2 * H + H + h] = (uint16_t)f2bf(acc - bf2f(hi));
}

hipError_t launch_fold_router(const uint16_t* D, const uint16_t* Wr, int E, int L, int H, uint16_t* Gr, hipStream_t s,
                              int Eg) {
    hipLaunchKernelGGL(fold_router_kernel, dim3((unsigned)cdiv(H, 256), (unsigned)E), dim3(256), 0, s, D, Wr, E, L, H,
                       Eg > 0 ? Eg : E, Gr);
    return last();
}

hipError_t launch_proj_partials(const uint16_t* xpart, int G, const uint16_t* W, int T, int N, int K, int mode, float* out32,
                                uint16_t* out16, hipStream_t s) {
    if (rows_proj_fits(T, K, 1, G))
        return rows_proj_launch<1>(
            RowsProj{xpart, nullptr, G, W, T, N, K, mode, out32, out16, nullptr, nullptr, nullptr, 0, nullptr, 0, 0.f}, s);
    if (!small_proj_fits(T, K)) return hipErrorInvalidValue;
    return small_proj_launch<1>(SmallProj{xpart, nullptr, G, W, T, N, K, mode, out32, out16, nullptr, nullptr, 0,
                                          nullptr, nullptr},
                                s);
}

// y = sum over the KG K groups of part[kg] (in order): mode 1: out16 = bf16(y); 2: out32 += y.
__global__ __launch_bounds__(256) void sum_groups_kernel(const float* __restrict__ part, int KG, int T, int N, int mode,
                                                         float* __restrict__ out32, uint16_t* __restrict__ out16) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x, n = (size_t)T * N;
    if (i >= n) return;
    float v = 0.f;
    for (int g = 0; g < KG; ++g) v += part[(size_t)g * n + i];
    if (mode == 2)
        out32[i] += v;
    else
        out16[i] = (uint16_t)f2bf(v);
}

hipError_t launch_proj_partials_kgroups(const uint16_t* xpart, int G, const uint16_t* W, int T, int N, int K, int KG,
                                        float* part, int mode, float* out32, uint16_t* out16, hipStream_t s) {
    if (!small_proj_fits(T, K)) return hipErrorInvalidValue;
    SmallProj p{xpart, nullptr, G, W, T, N, K, 3, part, nullptr, nullptr, nullptr, 0, nullptr, nullptr};
    p.KG = KG;
    hipError_t e = small_proj_launch<1>(p, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(sum_groups_kernel, dim3((unsigned)cdiv((size_t)T * N, 256)), dim3(256), 0, s, part, KG, T, N, mode,
                       out32, out16);
    return last();
}

hipError_t launch_proj_bf16(const uint16_t* x, const uint16_t* W, int T, int N, int K, int mode, float* out32,
                            uint16_t* out16, hipStream_t s, uint16_t* out16lo, uint16_t* out16h, const float* hnorm) {
    if (T <= kStreamMaxT && rows_proj_fits(T, K, hnorm ? 2 : 0) && mode != 3) {
        const RowsProj p{x, hnorm, 0, W, T, N, K, mode, out32, out16, out16h, nullptr, nullptr, 0, nullptr, 0, 0.f};
        return hnorm ? rows_proj_launch<2>(p, s) : rows_proj_launch<0>(p, s);
    }
    if (T <= kStreamMaxT && small_proj_fits(T, K)) {
        const SmallProj p{x, hnorm, 0, W, T, N, K, mode, out32, out16, nullptr, nullptr, 0, nullptr, out16h};
        return hnorm ? small_proj_launch<2>(p, s) : small_proj_launch<0>(p, s);
    }
    if (hnorm) return hipErrorInvalidValue;  // the caller normalises first for the other forms
    if (T <= kStreamMaxT)
        return launch_stream<kPW, kPKS, 1, StreamProj, kProjChunk>(StreamProj{x, W, T, N, K, mode, out32, out16},
                                                                   (int)cdiv(T, 16), N, s);
    if (LMOE_PIPE_PROJ) {
        // 256-row tiles halve the bytes per flop but come in half as many: take them when the
        // rounds of tiles over the CUs, weighted by a round of 256-row tiles' cost (kBigRoundCost),
        // come out lower
        const long nn = cdiv(N, PipeP::kBN), cus = cu_count();
        const long r1 = cdiv(cdiv(T, PipeP::kBM) * nn, cus), r2 = cdiv(cdiv(T, PipeB::kBM) * nn, cus);
        if (PipeB::kBN == PipeP::kBN && PipeB::kBM > PipeP::kBM && kBigRoundCost * r2 < 100 * r1) {
            PipeProj<PipeB> p{{x, W, T, N, K, mode, out32, out16, out16lo}};
            auto k = pipe_gemm_persistent<PipeB, PipeProj<PipeB>>;
            hipLaunchKernelGGL(k, dim3(std::min<long>(resident_blocks(k, PipeB::kThreads), (long)cdiv(T, PipeB::kBM) * nn)),
                               dim3(PipeB::kThreads), 0, s, p, (int)nn);
            return last();
        }
        PipeProj<PipeP> p{{x, W, T, N, K, mode, out32, out16, out16lo}};
        auto k = pipe_gemm_persistent<PipeP, PipeProj<PipeP>>;
        hipLaunchKernelGGL(k, dim3(std::min<long>(resident_blocks(k, PipeP::kThreads), (long)cdiv(T, PipeP::kBM) * nn)),
                           dim3(PipeP::kThreads), 0, s, p, (int)nn);
        return last();
    }
    TileProj<TileL> p{x, W, T, N, K, mode, out32, out16, out16lo};
    hipLaunchKernelGGL((tile_gemm_kernel<TileL, TileProj<TileL>>), dim3(cdiv(N, TileL::kBN), cdiv(T, TileL::kBM)),
                       dim3(256), 0, s, p);
    return last();
}

hipError_t launch_router_bf16(const float* z, const uint16_t* Wr, const float* br, int T, int E, int L, float* logits,
                              hipStream_t s, const uint16_t* zhi, const uint16_t* zlo) {
    if (T <= kStreamMaxT)
        return launch_stream<kPW, kPKS, 1, StreamRouter, kProjChunk>(StreamRouter{z, Wr, br, T, E, L, logits},
                                                                     (int)cdiv(T, 16), E, s);
    if (zhi && zlo) {
        // the two halves' logits: logits (hi, + br) and logits + T * E (lo); 256-row tiles when
        // their rounds over the CUs come out cheaper, by the projections' measured weighting
        const long nn = cdiv(E, PipeP::kBN), cus = cu_count();
        const long r1 = cdiv(2 * cdiv(T, PipeP::kBM) * nn, cus), r2 = cdiv(2 * cdiv(T, PipeB::kBM) * nn, cus);
        if (PipeB::kBN == PipeP::kBN && PipeB::kBM > PipeP::kBM && kBigRoundCost * r2 < 100 * r1) {
            PipeRouter<PipeB> p{zhi, zlo, Wr, br, T, E, L, logits};
            auto k = pipe_gemm_persistent<PipeB, PipeRouter<PipeB>>;
            hipLaunchKernelGGL(k, dim3(std::min<long>(resident_blocks(k, PipeB::kThreads), 2 * (long)cdiv(T, PipeB::kBM) * nn)),
                               dim3(PipeB::kThreads), 0, s, p, (int)nn);
            return last();
        }
        PipeRouter<PipeP> p{zhi, zlo, Wr, br, T, E, L, logits};
        auto k = pipe_gemm_persistent<PipeP, PipeRouter<PipeP>>;
        hipLaunchKernelGGL(k, dim3(std::min<long>(resident_blocks(k, PipeP::kThreads), 2 * (long)cdiv(T, PipeP::kBM) * nn)),
                           dim3(PipeP::kThreads), 0, s, p, (int)nn);
        return last();
    }
    TileRouter<TileL> p{z, Wr, br, T, E, L, logits, zhi, zlo};
    hipLaunchKernelGGL((tile_gemm_kernel<TileL, TileRouter<TileL>>), dim3(cdiv(E, TileL::kBN), cdiv(T, TileL::kBM)),
                       dim3(256), 0, s, p);
    return last();
}

// The router logits of a batch from x and the folded router Gr [E][2][K] (its rows as a [2E][K]
// matrix): logits[h][t][e] = x[t] . Gr[e][h] (+ br[e] for h = 0).
hipError_t launch_router_x(const uint16_t* x, const uint16_t* Gr, const float* br, int T, int E, int K, float* logits,
                           hipStream_t s) {
    TileProj<TileL> p{x, Gr, T, 2 * E, K, 3, logits, nullptr, nullptr, br};
    hipLaunchKernelGGL((tile_gemm_kernel<TileL, TileProj<TileL>>), dim3(cdiv(2 * E, TileL::kBN), cdiv(T, TileL::kBM)),
                       dim3(256), 0, s, p);
    return last();
}

hipError_t launch_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w, hipStream_t s,
                       const float* logits2) {
    const dim3 g(cdiv(T, 4)), b(256);
    if (E <= 64)
        hipLaunchKernelGGL(topk_kernel<1>, g, b, 0, s, logits, logits2, T, E, k, ids, w);
    else if (E <= 128)
        hipLaunchKernelGGL(topk_kernel<2>, g, b, 0, s, logits, logits2, T, E, k, ids, w);
    else if (E <= 256)
        hipLaunchKernelGGL(topk_kernel<4>, g, b, 0, s, logits, logits2, T, E, k, ids, w);
    else if (E <= 512)
        hipLaunchKernelGGL(topk_kernel<8>, g, b, 0, s, logits, logits2, T, E, k, ids, w);
    else
        hipLaunchKernelGGL(topk_kernel<16>, g, b, 0, s, logits, logits2, T, E, k, ids, w);
    return last();
}

int perm_blocks(int T) { return (int)cdiv(T, kPermTB); }

hipError_t launch_permute(const int32_t* ids, int T, int k, int E, int32_t* hist, int32_t* base, int32_t* offsets,
                          int32_t* perm, int32_t* inv, int BM, Tile* tiles, int32_t* ntiles, int has_shared, hipStream_t s) {
    const int nb = perm_blocks(T);
    if (nb <= 1) {
        hipLaunchKernelGGL(perm_single_kernel, dim3(1), dim3(1024), 0, s, ids, T, k, E, offsets, perm, inv, BM, tiles,
                           ntiles, has_shared);
        return last();
    }
    hipLaunchKernelGGL(perm_hist_kernel, dim3(nb), dim3(256), 0, s, ids, T, k, E, hist);
    hipError_t err = last();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(perm_scan_kernel, dim3(cdiv(E, kScanEPB)), dim3(1024), 0, s, hist, nb, E, base);
    err = last();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(perm_scatter_kernel, dim3(nb), dim3(256), 0, s, ids, T, k, E, nb, base, offsets, perm, inv, BM,
                       tiles, ntiles, has_shared);
    return last();
}

hipError_t launch_topk_permute(const float* logits, int T, int E, int k, int32_t* ids, float* w, int32_t* hist,
                               int32_t* base, int32_t* offsets, int32_t* perm, int32_t* inv, int BM, Tile* tiles,
                               int32_t* ntiles, int has_shared, hipStream_t s, const float* logits2, int2* rowinfo) {
    if (T > kPermTB) {
        if (rowinfo) return hipErrorInvalidValue;  // small-batch launch only
        hipError_t e = launch_topk(logits, T, E, k, ids, w, s, logits2);
        if (e != hipSuccess) return e;
        return launch_permute(ids, T, k, E, hist, base, offsets, perm, inv, BM, tiles, ntiles, has_shared, s);
    }
    const dim3 g(1), b(1024);
#define LMOE_TOPK_PERM(NV)                                                                                          \
    hipLaunchKernelGGL(topk_perm_single_kernel<NV>, g, b, 0, s, logits, logits2, T, E, k, ids, w, offsets, perm, inv, BM, \
                       tiles, ntiles, has_shared, rowinfo)
    if (E <= 64)
        LMOE_TOPK_PERM(1);
    else if (E <= 128)
        LMOE_TOPK_PERM(2);
    else if (E <= 256)
        LMOE_TOPK_PERM(4);
    else if (E <= 512)
        LMOE_TOPK_PERM(8);
    else
        LMOE_TOPK_PERM(16);
#undef LMOE_TOPK_PERM
    return last();
}

// 256-row tiles pay when segments fill them: a 256-row tile's second row of waves idles on a
// segment of at most 128 rows, while the tile still copies its weights whole.  They are taken
// when the average routed segment (T k / E rows) holds at least one such tile (measured: 16K
// tokens with Zipf(1.1) routing, 320 rows on average, 2.30 against 2.49 ms for 128-row tiles;
// 4096 uniformly routed tokens, 80 rows, 1.23 against 1.03 ms).
int expert_tile_rows(bool stream_path, bool mx_path, int T, int k, int E) {
    if (stream_path) return 16;
    if (mx_path) return PipeL::kBM;  // the block-scaled kernels' tile rows (checked with their shapes)
    if (!LMOE_PIPE) return TileL::kBM;
    const bool big = LMOE_PIPE_PERSIST && LMOE_BIG_TILES && (long)T * k >= (long)PipeB::kBM * E;
    return big ? PipeB::kBM : PipeL::kBM;
}

int expert_max_tiles(int T, int k, int E, int has_shared, bool stream_path, bool mx_path) {
    const long BM = expert_tile_rows(stream_path, mx_path, T, k, E);
    const long tk = (long)T * k;
    return (int)(cdiv(tk, BM) + std::min<long>(E, tk) + (has_shared ? cdiv(T, BM) : 0));
}

// Small-batch expert launches: gate/up work items of 16 columns dealt over one workgroup of
// LMOE_GU_WAVES waves per compute unit, then the down projection and merge over LMOE_DC_GROUPS
// groups of the work list.
constexpr int kGuWaves = LMOE_GU_WAVES, kGuChunk = LMOE_GU_CHUNK, kGuChunk4 = LMOE_GU_CHUNK4;
// K-split gate/up: largest runs of bf16 (32-value) and 4-bit (128-value) weight groups per wave
constexpr int kGuMG = 7, kGuMG4 = 2;
constexpr int kDcWaves = LMOE_DC_WAVES, kDcChunk = LMOE_DC_CHUNK, kDcChunk4 = LMOE_DC_CHUNK4, kDcGroups = LMOE_DC_GROUPS;

int decode_groups() { return kDcGroups; }

static_assert(16 * kSmallProjGroups >= kDecodeMaxT, "small-batch projections take every decode-path batch");

bool small_proj_fits(int T, int K) { return T <= 16 * kSmallProjGroups && small_proj_lds(K) <= kSmallProjLds; }

bool decode_fits(int T, int L, int F, int Fs) {
    // widths in whole 16-row blocks (a gate/up slice may end inside a segment); U stages its input in LDS
    return T <= kDecodeMaxT && F % 16 == 0 && Fs % 16 == 0 && small_proj_fits(T, L);
}

template <int Q>
hipError_t launch_decode_experts(const ExpertArgs& a, const SegSpace& seg, hipStream_t s, StageEvents& ev) {
    const int nblocks = (int)cdiv(a.Hs, 16);
    DecodeExperts<Q> d{seg,     a.z16, a.z16h, a.experts, a.rec_bytes, static_cast<const uint16_t*>(a.shared),
                       a.L,     a.F,   a.Fs,   a.Hs,      nblocks,     a.H,
                       a.w,     a.mpart, kDcGroups, a.rowinfo, a.max_tiles};
    const long items = (long)a.max_tiles * nblocks;
    // the gate/up stage's events are taken by the launch itself (kernel time only)
    hipEvent_t e0 = ev.start(kStageUp), e1 = ev.stop(kStageUp);
    // The K-split form when every wave's run of weight groups fits its registers and there are at
    // most as many items as waves on the chip (measured: at T = 1 it keeps all waves busy and
    // saves a fifth of the step; at T >= 8 one item per wave streams as fast or faster).
    const bool split = LMOE_GU_SPLIT && a.L / 32 <= kGuWaves * kGuMG &&
                       (Q == 0 || a.L / 128 <= kGuWaves * kGuMG4) && items <= (long)cu_count() * kGuWaves;
    const long grid = std::max<long>(std::min<long>(split ? items : cdiv(items, kGuWaves), cu_count()), 1);
    if (a.route) {  // the launch routes the batch itself (top-k and permutation in every workgroup)
        const GuRoute r{a.route->logits, a.route->logits2, a.route->BM, a.route->has_shared, a.route->out};
        const size_t lds = (size_t)a.max_tiles * sizeof(Tile);
        const int E = a.E;
#define LMOE_GU_ROUTED(NV)                                                                                          \
    if (split)                                                                                                      \
        hipExtLaunchKernelGGL((decode_gu_split_kernel<kGuWaves, kGuMG, kGuMG4, Q, NV>), dim3((unsigned)grid),      \
                              dim3(64 * kGuWaves), (uint32_t)lds, s, e0, e1, 0u, d, r);                             \
    else                                                                                                            \
        hipExtLaunchKernelGGL((decode_gu_kernel<kGuWaves, kGuChunk, kGuChunk4, Q, NV>), dim3((unsigned)grid),      \
                              dim3(64 * kGuWaves), (uint32_t)lds, s, e0, e1, 0u, d, r)
        if (E <= 64)
            LMOE_GU_ROUTED(1);
        else if (E <= 128)
            LMOE_GU_ROUTED(2);
        else if (E <= 256)
            LMOE_GU_ROUTED(4);
        else if (E <= 512)
            LMOE_GU_ROUTED(8);
        else
            LMOE_GU_ROUTED(16);
#undef LMOE_GU_ROUTED
    } else if (split) {
        hipExtLaunchKernelGGL((decode_gu_split_kernel<kGuWaves, kGuMG, kGuMG4, Q, 0>), dim3((unsigned)grid),
                              dim3(64 * kGuWaves), 0u, s, e0, e1, 0u, d, GuRoute{});
    } else {
        hipExtLaunchKernelGGL((decode_gu_kernel<kGuWaves, kGuChunk, kGuChunk4, Q, 0>), dim3((unsigned)grid),
                              dim3(64 * kGuWaves), 0u, s, e0, e1, 0u, d, GuRoute{});
    }
    hipError_t err = last();
    if (err != hipSuccess) return err;
    ev.begin(kStageDown);
    const size_t lds =
        (size_t)a.max_tiles * sizeof(Tile) + (size_t)a.T * a.k * sizeof(int2) + (size_t)a.max_tiles * sizeof(int);
    const unsigned xgroups = (unsigned)(seg.zp / a.L);
    hipLaunchKernelGGL((decode_dc_kernel<kDcWaves, kDcChunk, kDcChunk4, Q>), dim3(a.L / 16, kDcGroups, xgroups),
                       dim3(64 * kDcWaves), lds, s, d);
    if ((err = last()) != hipSuccess) return err;
    ev.end(kStageDown);
    return hipSuccess;
}

// Large 4-bit batches: the records of the experts that received tokens are decoded once into
// packed bf16 records (the exact values: an E2M1 value times an E8M0 or E4M3 block scale has at
// most 6 significant bits), and the bf16 pipelined GEMMs run on them; an NVFP4 record's fp32
// tensor scales go to ts [E][3] and multiply the products in the epilogues.
// Thread u of expert blockIdx.y decodes 16-byte unit u of the record (gate, up, then down): 32
// values of one row, which are four bf16 units of the bf16 tile holding the same columns.
template <int Q>
__global__ __launch_bounds__(256) void dequant_experts_kernel(const uint8_t* __restrict__ src, size_t rec4,
                                                              const int32_t* __restrict__ offsets, int F, int L,
                                                              uint16_t* __restrict__ dst, float* __restrict__ ts) {
    const int e = blockIdx.y;
    if (offsets[e + 1] == offsets[e]) return;  // no tokens: the record is not read
    constexpr int kSB = Q == 1 ? 1 : 2;
    const size_t FL = (size_t)F * L, upm = FL / 32;  // units per matrix
    const uint8_t* rec = src + (size_t)e * rec4;
    uint16_t* out = dst + (size_t)e * 3 * FL;
    if (blockIdx.x == 0 && threadIdx.x < 3)
        ts[3 * e + threadIdx.x] = Q == 2 ? reinterpret_cast<const float*>(rec + 3 * (FL / 2) + 3 * (FL / 16))[threadIdx.x] : 1.f;
    const size_t u = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (u >= 3 * upm) return;
    const int m = (int)(u / upm);
    const size_t v = u - (size_t)m * upm;
    const int K = m < 2 ? L : F;                       // gate/up [F][L], down [L][F]
    const int gpr = K / 128;                           // 128-value groups per row block
    const size_t rb = v / ((size_t)gpr * 64);
    const int rem = (int)(v - rb * gpr * 64), g = rem >> 6, pos = rem & 63, q4 = pos >> 4, j = pos & 15;
    const uint4 nib = *reinterpret_cast<const uint4*>(rec + (size_t)m * (FL / 2) + rb * 8 * K + g * 1024 + pos * 16);
    const uint8_t* sp = rec + 3 * (FL / 2) + ((size_t)m * upm + (rb * gpr + g) * 64 + pos) * kSB;
    float s0, s1;
    if constexpr (Q == 1) {
        s0 = s1 = e8m0_to_f32(*sp);
    } else {
        s0 = e4m3_to_f32(sp[0]);
        s1 = e4m3_to_f32(sp[1]);
    }
    uint16_t* o = out + (size_t)m * FL + rb * 16 * K + (size_t)(g * 4 + q4) * 512 + j * 8;
    const uint32_t w[4] = {nib.x, nib.y, nib.z, nib.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) *reinterpret_cast<uint4*>(o + q * 128) = fp4x8_to_bf16x8(w[q], q < 2 ? s0 : s1);
}

hipError_t launch_dequant_experts(const void* src, size_t rec4, const int32_t* offsets, int E, int F, int L, int fmt,
                                  uint16_t* dst, float* ts, hipStream_t s) {
    const dim3 grid((unsigned)cdiv((size_t)3 * F * L / 32, 256), (unsigned)E);
    if (fmt == 2)
        hipLaunchKernelGGL(dequant_experts_kernel<2>, grid, dim3(256), 0, s, static_cast<const uint8_t*>(src), rec4,
                           offsets, F, L, dst, ts);
    else
        hipLaunchKernelGGL(dequant_experts_kernel<1>, grid, dim3(256), 0, s, static_cast<const uint8_t*>(src), rec4,
                           offsets, F, L, dst, ts);
    return last();
}

// Larger 4-bit batches: persistent weight-streaming gate/up, then down (the combine follows).
template <int Q>
hipError_t launch_stream_experts(const ExpertArgs& a, const SegSpace& seg, hipStream_t s, StageEvents& ev) {
    const int Fmax = std::max(a.F, a.Fs);
    const uint16_t* sh = static_cast<const uint16_t*>(a.shared);
    ev.begin(kStageUp);
    hipError_t err = launch_stream<kUW, kUKS, 2>(StreamUp<Q>{seg, a.z16, a.experts, a.rec_bytes, sh, a.L, a.F, a.Fs,
                                                              a.Hs, a.H},
                                                 a.max_tiles, Fmax, s);
    if (err != hipSuccess) return err;
    ev.end(kStageUp);
    ev.begin(kStageDown);
    err = launch_stream<kDW, kDKS, 1>(StreamDown<Q>{seg, a.H, a.experts, a.rec_bytes, sh, a.L, a.F, a.Fs, a.Hs, a.Y},
                                      a.max_tiles, a.L, s);
    if (err != hipSuccess) return err;
    ev.end(kStageDown);
    return hipSuccess;
}

// Large MXFP4 batches on the block-scaled MFMA: z to MXFP8 plus an MXFP4 residual, the routed
// gate/up product (H in bf16), H to MXFP8 plus an MXFP4 residual, and the down product, both
// products from the stored records; the shared expert's (bf16) segment takes the bf16 kernels.
// LMOE_MX_H_LO=0 builds the down product without H's residual term (for measurement).
#ifndef LMOE_MX_NS_UP
#define LMOE_MX_NS_UP 2
#endif
#ifndef LMOE_MX_NS_DN
#define LMOE_MX_NS_DN 3
#endif
using MxUpL = MxShape<128, 256, LMOE_MX_NS_UP, 2, 4, true>;
#ifndef LMOE_MX_H_LO
#define LMOE_MX_H_LO 1
#endif
using MxDnL = MxShape<128, 256, LMOE_MX_NS_DN, 2, 4, LMOE_MX_H_LO != 0>;
static_assert(MxUpL::kBM == PipeL::kBM && MxDnL::kBM == PipeL::kBM, "the work list's tile rows");

hipError_t launch_experts_mx(const ExpertArgs& a, const SegSpace& seg, hipStream_t s, StageEvents& ev) {
    if (!a.z8 || !a.z8s || !a.z4 || !a.z4s || !a.h8 || !a.h8s || !a.h16 || (MxDnL::kLo && (!a.h4 || !a.h4s)) ||
        a.fmt != 1 || a.L % 128 || a.F % 128)
        return hipErrorInvalidValue;
    const int nsh = a.shared ? (int)cdiv(a.T, MxUpL::kBM) : 0;
    SegSpace rs = seg;
    rs.part = 1;
    rs.nsh = nsh;
    SegSpace ss = rs;
    ss.part = 2;
    const uint8_t* ex = static_cast<const uint8_t*>(a.experts);
    const uint16_t* sh = static_cast<const uint16_t*>(a.shared);
    const int zp = a.zp > 0 ? a.zp : a.L;
    ev.begin(kStageUp);
    const size_t nblk = (size_t)a.T * zp / 32;
    hipLaunchKernelGGL(quant_mx_kernel, dim3((unsigned)cdiv(nblk, 256)), dim3(256), 0, s, a.z16, nblk, a.z8, a.z8s,
                       a.z4, a.z4s);
    hipError_t err = last();
    if (err != hipSuccess) return err;
    {
        MxUp<MxUpL> up{rs, a.z8, a.z8s, a.z4, a.z4s, ex, a.rec_bytes, a.L, a.F, a.h16};
        const int nn = (int)cdiv(a.F, MxUpL::kBN / 2);
        auto k = mx_gemm_persistent<MxUpL, MxUp<MxUpL>>;
        hipLaunchKernelGGL(k, dim3(std::min<long>(resident_blocks(k, MxUpL::kThreads), (long)a.max_tiles * nn)),
                           dim3(MxUpL::kThreads), 0, s, up, nn);
        if ((err = last()) != hipSuccess) return err;
    }
    if (nsh > 0) {
        PipeUp<PipeL> up{{ss, a.z16, sh, sh, 0, a.L, a.F, a.Fs, a.Hs, a.H, nullptr}};
        const int nn = (int)cdiv(a.Fs, PipeL::kBN / 2);
        auto k = pipe_gemm_persistent<PipeL, PipeUp<PipeL>>;
        hipLaunchKernelGGL(k, dim3(std::min<long>(resident_blocks(k, PipeL::kThreads), (long)nsh * nn)),
                           dim3(PipeL::kThreads), 0, s, up, nn);
        if ((err = last()) != hipSuccess) return err;
    }
    ev.end(kStageUp);
    ev.begin(kStageDown);
    const size_t hblk = (size_t)a.T * a.k * a.F / 32;  // the routed rows of H
    hipLaunchKernelGGL(quant_mx_kernel, dim3((unsigned)cdiv(hblk, 256)), dim3(256), 0, s, a.h16, hblk, a.h8, a.h8s,
                       MxDnL::kLo ? a.h4 : nullptr, a.h4s);
    if ((err = last()) != hipSuccess) return err;
    {
        MxDown<MxDnL> dn{rs, a.h8, a.h8s, a.h4, a.h4s, ex, a.rec_bytes, a.L, a.F, a.Y};
        const int nn = (int)cdiv(a.L, MxDnL::kBN);
        auto k = mx_gemm_persistent<MxDnL, MxDown<MxDnL>>;
        hipLaunchKernelGGL(k, dim3(std::min<long>(resident_blocks(k, MxDnL::kThreads), (long)a.max_tiles * nn)),
                           dim3(MxDnL::kThreads), 0, s, dn, nn);
        if ((err = last()) != hipSuccess) return err;
    }
    if (nsh > 0) {
        PipeDown<PipeL> dn{{ss, a.H, sh, sh, 0, a.L, a.F, a.Fs, a.Hs, a.Y, nullptr}};
        const int nn = (int)cdiv(a.L, PipeL::kBN);
        auto k = pipe_gemm_persistent<PipeL, PipeDown<PipeL>>;
        hipLaunchKernelGGL(k, dim3(std::min<long>(resident_blocks(k, PipeL::kThreads), (long)nsh * nn)),
                           dim3(PipeL::kThreads), 0, s, dn, nn);
        if ((err = last()) != hipSuccess) return err;
    }
    ev.end(kStageDown);
    return hipSuccess;
}

hipError_t launch_experts_bf16(const ExpertArgs& a, hipStream_t s, StageEvents& ev) {
    const SegSpace seg{a.tiles, a.ntiles, a.perm, a.T, a.k, a.E, a.Eg > 0 ? a.Eg : a.E, a.zp > 0 ? a.zp : a.L};
    if (a.decode_path)
        return a.fmt == 2 ? launch_decode_experts<2>(a, seg, s, ev)
                          : a.fmt == 1 ? launch_decode_experts<1>(a, seg, s, ev) : launch_decode_experts<0>(a, seg, s, ev);
    if (a.stream_path)
        return a.fmt == 2 ? launch_stream_experts<2>(a, seg, s, ev)
                          : a.fmt == 1 ? launch_stream_experts<1>(a, seg, s, ev) : launch_stream_experts<0>(a, seg, s, ev);
    if (a.mx_path) return launch_experts_mx(a, seg, s, ev);
    // the tile path takes bf16 records: a 4-bit layer's are decoded first into a.deq
    const uint16_t* ex = static_cast<const uint16_t*>(a.experts);
    size_t rec = a.rec_bytes / 2;
    ev.begin(kStageUp);  // the decode of 4-bit records counts to the gate/up stage
    if (a.fmt != 0) {
        if (!a.deq || !a.deq_ts) return hipErrorInvalidValue;
        hipError_t err = launch_dequant_experts(a.experts, a.rec_bytes, a.offsets, a.E, a.F, a.L, a.fmt, a.deq, a.deq_ts, s);
        if (err != hipSuccess) return err;
        ex = a.deq;
        rec = (size_t)3 * a.F * a.L;
    }
    const float* tsc = a.fmt != 0 ? a.deq_ts : nullptr;
    const int Fmax = std::max(a.F, a.Fs);
    const uint16_t* sh = static_cast<const uint16_t*>(a.shared);
    if (LMOE_PIPE && LMOE_PIPE_PERSIST && a.tile_rows == PipeB::kBM) {  // 256-row tiles (expert_tile_rows)
        const int nn_up = (int)cdiv(Fmax, PipeB::kBN / 2), nn_dn = (int)cdiv(a.L, PipeB::kBN);
        auto ku = pipe_gemm_persistent<PipeB, PipeUp<PipeB>>;
        hipLaunchKernelGGL(ku, dim3(std::min<long>(resident_blocks(ku, PipeB::kThreads), (long)a.max_tiles * nn_up)),
                           dim3(PipeB::kThreads), 0, s, PipeUp<PipeB>{{seg, a.z16, ex, sh, rec, a.L, a.F, a.Fs, a.Hs, a.H, tsc}},
                           nn_up);
        hipError_t err = last();
        if (err != hipSuccess) return err;
        ev.end(kStageUp);
        ev.begin(kStageDown);
        auto kd = pipe_gemm_persistent<PipeB, PipeDown<PipeB>>;
        hipLaunchKernelGGL(kd, dim3(std::min<long>(resident_blocks(kd, PipeB::kThreads), (long)a.max_tiles * nn_dn)),
                           dim3(PipeB::kThreads), 0, s,
                           PipeDown<PipeB>{{seg, a.H, ex, sh, rec, a.L, a.F, a.Fs, a.Hs, a.Y, tsc}}, nn_dn);
        if ((err = last()) != hipSuccess) return err;
        ev.end(kStageDown);
        return hipSuccess;
    }
    if (LMOE_PIPE) {
        PipeUp<PipeL> up{{seg, a.z16, ex, sh, rec, a.L, a.F, a.Fs, a.Hs, a.H, tsc}};
        const int nn_up = (int)cdiv(Fmax, PipeL::kBN / 2);
        if (LMOE_PIPE_PERSIST) {
            auto k = pipe_gemm_persistent<PipeL, PipeUp<PipeL>>;
            hipLaunchKernelGGL(k, dim3(std::min<long>(resident_blocks(k, PipeL::kThreads), (long)a.max_tiles * nn_up)), dim3(PipeL::kThreads), 0,
                               s, up, nn_up);
        } else {
            hipLaunchKernelGGL((pipe_gemm_kernel<PipeL, PipeUp<PipeL>>), dim3(nn_up, a.max_tiles), dim3(PipeL::kThreads), 0, s, up);
        }
        hipError_t err = last();
        if (err != hipSuccess) return err;
        ev.end(kStageUp);
        ev.begin(kStageDown);
        PipeDown<PipeL> dn{{seg, a.H, ex, sh, rec, a.L, a.F, a.Fs, a.Hs, a.Y, tsc}};
        const int nn_dn = (int)cdiv(a.L, PipeL::kBN);
        if (LMOE_PIPE_PERSIST) {
            auto k = pipe_gemm_persistent<PipeL, PipeDown<PipeL>>;
            hipLaunchKernelGGL(k, dim3(std::min<long>(resident_blocks(k, PipeL::kThreads), (long)a.max_tiles * nn_dn)), dim3(PipeL::kThreads), 0,
                               s, dn, nn_dn);
        } else {
            hipLaunchKernelGGL((pipe_gemm_kernel<PipeL, PipeDown<PipeL>>), dim3(nn_dn, a.max_tiles), dim3(PipeL::kThreads), 0, s, dn);
        }
        if ((err = last()) != hipSuccess) return err;
        ev.end(kStageDown);
        return hipSuccess;
    }
    TileUp<TileL> up{seg, a.z16, ex, sh, rec, a.L, a.F, a.Fs, a.Hs, a.H, tsc};
    hipLaunchKernelGGL((tile_gemm_kernel<TileL, TileUp<TileL>>), dim3(cdiv(Fmax, TileL::kBN / 2), a.max_tiles),
                       dim3(256), 0, s, up);
    hipError_t err = last();
    if (err != hipSuccess) return err;
    ev.end(kStageUp);
    ev.begin(kStageDown);
    TileDown<TileL> dn{seg, a.H, ex, sh, rec, a.L, a.F, a.Fs, a.Hs, a.Y, tsc};
    hipLaunchKernelGGL((tile_gemm_kernel<TileL, TileDown<TileL>>), dim3(cdiv(a.L, TileL::kBN), a.max_tiles),
                       dim3(256), 0, s, dn);
    if ((err = last()) != hipSuccess) return err;
    ev.end(kStageDown);
    return hipSuccess;
}


hipError_t launch_combine(const void* Y, const float* w, int T, int k, int L, int has_shared, bool out_bf16, void* m,
                          hipStream_t s, const int32_t* ids, int groups, int Eg) {
    const dim3 grid(cdiv(L / 8, 256), std::min(T, 65535), groups > 1 ? groups : 1);
    const int32_t* gids = groups > 1 ? ids : nullptr;
    if (out_bf16)
        hipLaunchKernelGGL(combine_kernel<true>, grid, dim3(256), 0, s, Y, w, T, k, L, has_shared, m, gids, Eg);
    else
        hipLaunchKernelGGL(combine_kernel<false>, grid, dim3(256), 0, s, Y, w, T, k, L, has_shared, m, gids, Eg);
    return last();
}

hipError_t launch_proj_f32(const float* x, const float* W, const float* bias, int T, int N, int K, int mode, float* out,
                           hipStream_t s) {
    hipLaunchKernelGGL(f32_proj_kernel, dim3(cdiv(N, 256), std::min(T, 65535)), dim3(256), 0, s, x, W, bias, T, N, K,
                       mode, out);
    return last();
}

hipError_t launch_experts_f32(const F32ExpertArgs& a, hipStream_t s, StageEvents& ev) {
    const F32Seg seg{a.z, a.ids, a.perm, a.experts, a.shared, a.T, a.k, a.L, a.F, a.Fs, a.Hs};
    const int R = a.T * a.k + (a.Fs > 0 ? a.T : 0);
    const int gy = std::min(R, 65535);
    ev.begin(kStageUp);
    hipLaunchKernelGGL(f32_up_kernel, dim3(cdiv(std::max(a.F, a.Fs), 256), gy), dim3(256), 0, s, seg, R, a.H);
    hipError_t err = last();
    if (err != hipSuccess) return err;
    ev.end(kStageUp);
    ev.begin(kStageDown);
    hipLaunchKernelGGL(f32_down_kernel, dim3(cdiv(a.L, 256), gy), dim3(256), 0, s, seg, R, a.H, a.Y);
    err = last();
    ev.end(kStageDown);
    return err;
}

}  // namespace lmoe
