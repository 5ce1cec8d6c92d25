// Problem definitions plugged into the tile (prefill) and stream (decode) MFMA kernels.
//
// Row spaces used by the expert kernels: the R = T*k (+ T when a shared expert exists)
// "segment rows".  Rows [0, T*k) are the routed (token, slot) pairs in permutation order,
// so expert e owns rows [offsets[e], offsets[e+1]); row p stands for slot perm[p], i.e.
// token perm[p] / k.  Rows [T*k, T*k + T) are the shared expert's segment, row T*k + t
// standing for token t.  H (SwiGLU hidden) is stored by segment row; Y (expert outputs) is
// stored token-major: row perm[p] = t*k + s for routed rows, T*k + t for shared rows, so
// the combine reads each token's contributions contiguously.
#pragma once

#include "common.hpp"
#include "gemm_tile.hpp"

namespace lmoe {

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
// Non-temporal 16-byte load, for data streamed once per step: the expert weight rows of the
// small-batch kernels (gate/up and down).  Plain loads of those rows left the caches to them and
// pushed out what the step reads again (decode_t8: gate/up 37.8 -> 34.7 us, down 20.0 -> 19.1 us,
// step 73 -> 68 us); the D and U projections' rows gained nothing from it and keep plain loads.
__device__ __forceinline__ uint4 ld16_nt(const void* p) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
#ifndef LMOE_WEIGHT_NT
#define LMOE_WEIGHT_NT 1
#endif
#if LMOE_WEIGHT_NT
#define LMOE_WLOAD ld16_nt
#else
#define LMOE_WLOAD ld16
#endif
__device__ __forceinline__ uint4 zero4() { return make_uint4(0, 0, 0, 0); }

// 8 consecutive fp32 values -> hi (lo = false) or lo (lo = true) halves as 8 bf16.
__device__ __forceinline__ uint4 f32x8_to_bf16_part(const float* src, bool lo) {
    const float4 a = *reinterpret_cast<const float4*>(src);
    const float4 b = *reinterpret_cast<const float4*>(src + 4);
    const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t h0, l0, h1, l1;
        split_hi_lo(v[2 * i], h0, l0);
        split_hi_lo(v[2 * i + 1], h1, l1);
        o[i] = lo ? (l0 | (l1 << 16)) : (h0 | (h1 << 16));
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
}

// Shared description of the grouped (per-expert) row space.
struct SegSpace {
    const Tile* tiles;      // work list
    const int32_t* ntiles;  // number of valid entries
    const int32_t* perm;    // [T*k]
    int32_t T, k, E;
    // Expert groups with their own D: z is [T][zp] with group g's latent in columns g*L ..;
    // expert seg is in group seg / Eg, the shared expert in group 0 (one group: Eg = E, zp = L).
    int32_t Eg, zp;
    // which tiles of the list a launch takes: 0 all, 1 the routed ones, 2 the shared segment's
    // (the last nsh entries of the list)
    int32_t part = 0, nsh = 0;
    __device__ __forceinline__ int count() const { return part == 0 ? *ntiles : part == 1 ? *ntiles - nsh : nsh; }
    __device__ __forceinline__ Tile at(int i) const { return tiles[part == 2 ? *ntiles - nsh + i : i]; }
    // a dropped slot (perm = -1) maps to token 0: its rows are computed but never stored
    __device__ __forceinline__ int token_of(int seg, int p) const { return seg == E ? p - T * k : max(perm[p], 0) / k; }
    __device__ __forceinline__ int dest_of(int seg, int p) const { return seg == E ? p : perm[p]; }
    // element offset of segment row p's token operand in z (latent width L)
    __device__ __forceinline__ size_t z_off(int seg, int tok, int L) const {
        return (size_t)tok * zp + (seg == E ? 0 : (size_t)(seg / Eg) * L);
    }
};

// =============================================================================================
// Tile (prefill) problems: 128x128 tiles, 2x2 waves of 64x64.
// =============================================================================================
using Tile128 = TileShape<128, 128, 2, 2>;
using Tile256 = TileShape<256, 256, 2, 2>;

// Dense projection C[t][n] = x[t] . W[n]; mode 0: z32 (optional) + z16 (D), 1: bf16 y (U), 2: y += (U, fp32
// residual), 3: router halves from the folded router (W = Gr as [2E][K] rows, n = 2e + h):
// out32[h][t][e] = v (+ bias[e] for h = 0)
template <class S>
struct TileProj {
    const uint16_t* x;  // [M][K] bf16
    const uint16_t* W;  // [N][K] bf16
    int M, N, K, mode;
    float* out32;
    uint16_t* out16;
    uint16_t* out16lo;  // mode 0, optional: bf16(v - bf16(v)), the low half of the router input
    const float* bias = nullptr;  // mode 3
    struct Ctx { int m0, n0; };
    typedef const uint16_t* RowA;
    typedef const uint16_t* RowB;
    __device__ bool tile(int bx, int by, Ctx& c) const {
        c.m0 = bx * S::kBM;
        c.n0 = by * S::kBN;
        return c.m0 < M && c.n0 < N;
    }
    __device__ RowA row_a(const Ctx& c, int r) const { return c.m0 + r < M ? x + (size_t)(c.m0 + r) * K : nullptr; }
    __device__ RowB row_b(const Ctx& c, int r) const { return c.n0 + r < N ? W + (size_t)(c.n0 + r) * K : nullptr; }
    __device__ int k_tiles(const Ctx&) const { return K / 64; }
    __device__ uint4 load_a(const Ctx&, RowA r, int kt, int lc) const { return r ? ld16(r + kt * 64 + lc * 8) : zero4(); }
    __device__ uint4 load_b(const Ctx&, RowB r, int kt, int lc) const { return r ? ld16(r + kt * 64 + lc * 8) : zero4(); }
    template <int MB, int NB>
    __device__ __forceinline__ void epilogue(const Ctx& c, f32x16 (&acc)[MB][NB], int rb, int cb, int lane) const {
        static_for<MB>([&](auto i) {
            static_for<NB>([&](auto j) {
                __builtin_amdgcn_sched_barrier(0);  // one block at a time (bounded registers)
                const int n = c.n0 + cb + j * 32 + frag32_col(lane);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = c.m0 + rb + i * 32 + frag32_row(r, lane);
                    if (m < M && n < N) {
                        const float v = acc[i][j][r];
                        const size_t o = (size_t)m * N + n;
                        if (mode == 0) {
                            uint32_t hi, lo;
                            split_hi_lo(v, hi, lo);
                            if (out32) out32[o] = v;
                            out16[o] = (uint16_t)hi;
                            if (out16lo) out16lo[o] = (uint16_t)lo;
                        } else if (mode == 3) {
                            const int e = n >> 1, h = n & 1;
                            out32[((size_t)h * M + m) * (N >> 1) + e] = h == 0 && bias ? v + bias[e] : v;
                        } else if (mode == 1) {
                            out16[o] = (uint16_t)f2bf(v);
                        } else {
                            out32[o] += v;
                        }
                    }
                }
            });
        });
    }
};

// Router logits from fp32 z: K doubled, first half multiplies hi(z), second half lo(z), same Wr.
// The halves are read from zhi/zlo when given (written by the D projection), else split from z.
template <class S>
struct TileRouter {
    const float* z;      // [M][K] fp32
    const uint16_t* W;   // [E][K] bf16
    const float* bias;   // [E] or null
    int M, N, K;
    float* logits;       // [M][N]
    const uint16_t* zhi;  // [M][K] bf16(z), or null
    const uint16_t* zlo;  // [M][K] bf16(z - bf16(z)), or null
    struct Ctx { int m0, n0; };
    typedef int RowA;  // row index, -1 outside
    typedef const uint16_t* RowB;
    __device__ bool tile(int bx, int by, Ctx& c) const {
        c.m0 = bx * S::kBM;
        c.n0 = by * S::kBN;
        return c.m0 < M && c.n0 < N;
    }
    __device__ RowA row_a(const Ctx& c, int r) const { return c.m0 + r < M ? c.m0 + r : -1; }
    __device__ RowB row_b(const Ctx& c, int r) const { return c.n0 + r < N ? W + (size_t)(c.n0 + r) * K : nullptr; }
    __device__ int k_tiles(const Ctx&) const { return 2 * (K / 64); }
    __device__ uint4 load_a(const Ctx&, RowA r, int kt, int lc) const {
        if (r < 0) return zero4();
        const int h = K / 64;
        const bool lo = kt >= h;
        const size_t o = (size_t)r * K + (lo ? kt - h : kt) * 64 + lc * 8;
        if (zhi) return ld16((lo ? zlo : zhi) + o);
        return f32x8_to_bf16_part(z + o, lo);
    }
    __device__ uint4 load_b(const Ctx&, RowB r, int kt, int lc) const {
        if (!r) return zero4();
        const int h = K / 64;
        return ld16(r + (kt >= h ? kt - h : kt) * 64 + lc * 8);
    }
    template <int MB, int NB>
    __device__ __forceinline__ void epilogue(const Ctx& c, f32x16 (&acc)[MB][NB], int rb, int cb, int lane) const {
        static_for<MB>([&](auto i) {
            static_for<NB>([&](auto j) {
                const int n = c.n0 + cb + j * 32 + frag32_col(lane);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = c.m0 + rb + i * 32 + frag32_row(r, lane);
                    if (m < M && n < N) logits[(size_t)m * N + n] = acc[i][j][r] + (bias ? bias[n] : 0.f);
                }
            });
        });
    }
};

// Expert matrices are stored packed (written by lmoe_pack_experts): a bf16 [N][K] matrix is a
// sequence of 1 KB tiles, 16 rows x 32 columns each, ordered by (row block, column step); inside
// a tile the 16-byte unit of row j, columns 8 q .. 8 q + 7 sits at position 16 q + j.  That is
// the register image of a v_mfma_f32_16x16x32_bf16 A operand, so a wave loads it with one
// contiguous 1 KB access.  packed_row gives row n's first unit, packed_chunk the unit holding
// columns 64 kt + 8 lc .. + 7.
__device__ __forceinline__ const uint16_t* packed_row(const uint16_t* m, int n, int K) {
    return m + (size_t)(n >> 4) * 16 * K + (n & 15) * 8;
}
__device__ __forceinline__ const uint16_t* packed_chunk(const uint16_t* row, int kt, int lc) {
    return row + (kt * 2 + (lc >> 2)) * 512 + (lc & 3) * 128;
}

// Fused SwiGLU gate/up over a work list.  The B tile's rows are, for each wave column of kWN
// rows, kWN/2 gate rows followed by the same kWN/2 up rows, so every lane ends with g and u of
// the same (row, f) in acc[i][j] / acc[i][j + NB/2] and applies SiLU(g) * u in registers.
template <class S>
struct TileUp {
    static constexpr int kHalf = S::kWN / 2;        // f per wave column
    static constexpr int kFPerTile = S::kBN / 2;    // f per tile
    SegSpace seg;
    const uint16_t* z16;      // [T][L]
    const uint16_t* experts;  // E records
    const uint16_t* shared;   // record or null
    size_t rec;               // elements per routed record
    int L, F, Fs, Hs;
    uint16_t* H;              // [R][Hs]
    const float* ts = nullptr;  // [E][3] tensor scales of the routed records (gate, up, down), or null (1)
    struct Ctx { int seg, row0, nrows, F, f0; const uint16_t* g; const uint16_t* u; float tg, tu; };
    typedef const uint16_t* RowA;
    typedef const uint16_t* RowB;
    __device__ bool tile(int bx, int by, Ctx& c) const {
        if (bx >= seg.count()) return false;
        const Tile t = seg.at(bx);
        c.seg = t.seg;
        c.row0 = t.row0;
        c.nrows = t.nrows;
        c.tg = c.tu = 1.f;
        if (t.seg == seg.E) {
            c.F = Fs;
            c.g = shared;
        } else {
            c.F = F;
            c.g = experts + (size_t)t.seg * rec;
            if (ts) {
                c.tg = ts[3 * t.seg];
                c.tu = ts[3 * t.seg + 1];
            }
        }
        c.u = c.g + (size_t)c.F * L;
        c.f0 = by * kFPerTile;
        return c.f0 < c.F;
    }
    __device__ RowA row_a(const Ctx& c, int r) const {
        if (r >= c.nrows) return nullptr;
        return z16 + seg.z_off(c.seg, seg.token_of(c.seg, c.row0 + r), L);
    }
    __device__ RowB row_b(const Ctx& c, int r) const {
        const int wc = r / S::kWN, rr = r % S::kWN;
        const int f = c.f0 + wc * kHalf + rr % kHalf;
        if (f >= c.F) return nullptr;
        return packed_row(rr >= kHalf ? c.u : c.g, f, L);
    }
    __device__ int k_tiles(const Ctx&) const { return L / 64; }
    __device__ uint4 load_a(const Ctx&, RowA r, int kt, int lc) const { return r ? ld16(r + kt * 64 + lc * 8) : zero4(); }
    __device__ uint4 load_b(const Ctx&, RowB r, int kt, int lc) const { return r ? ld16(packed_chunk(r, kt, lc)) : zero4(); }
    template <int MB, int NB>
    __device__ __forceinline__ void epilogue(const Ctx& c, f32x16 (&acc)[MB][NB], int rb, int cb, int lane) const {
        static_assert(NB % 2 == 0 && NB * 16 == kHalf, "gate blocks then up blocks per wave column");
        static_for<NB / 2>([&](auto j) {
            const int f = c.f0 + (cb / S::kWN) * kHalf + j * 32 + frag32_col(lane);
            static_for<MB>([&](auto i) {
                __builtin_amdgcn_sched_barrier(0);  // one block at a time (bounded registers)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = rb + i * 32 + frag32_row(r, lane);
                    if (m < c.nrows && f < c.F)
                        H[(size_t)(c.row0 + m) * Hs + f] =
                            (uint16_t)f2bf(silu(acc[i][j][r] * c.tg) * (acc[i][j + NB / 2][r] * c.tu));
                }
            });
        });
    }
};

// Down projection over a work list: Y[dest(p)][n] = H[p] . down[n].
template <class S>
struct TileDown {
    SegSpace seg;
    const uint16_t* H;
    const uint16_t* experts;
    const uint16_t* shared;
    size_t rec;
    int L, F, Fs, Hs;
    uint16_t* Y;  // [R][L] bf16
    const float* ts = nullptr;  // [E][3] tensor scales of the routed records, or null (1)
    struct Ctx { int seg, row0, nrows, F, n0; const uint16_t* d; float td; };
    typedef const uint16_t* RowA;
    typedef const uint16_t* RowB;
    __device__ bool tile(int bx, int by, Ctx& c) const {
        if (bx >= seg.count()) return false;
        const Tile t = seg.at(bx);
        c.seg = t.seg;
        c.row0 = t.row0;
        c.nrows = t.nrows;
        c.td = 1.f;
        if (t.seg == seg.E) {
            c.F = Fs;
            c.d = shared + 2 * (size_t)Fs * L;
        } else {
            c.F = F;
            c.d = experts + (size_t)t.seg * rec + 2 * (size_t)F * L;
            if (ts) c.td = ts[3 * t.seg + 2];
        }
        c.n0 = by * S::kBN;
        return c.n0 < L;
    }
    __device__ RowA row_a(const Ctx& c, int r) const { return r < c.nrows ? H + (size_t)(c.row0 + r) * Hs : nullptr; }
    __device__ RowB row_b(const Ctx& c, int r) const { return c.n0 + r < L ? packed_row(c.d, c.n0 + r, c.F) : nullptr; }
    __device__ int k_tiles(const Ctx& c) const { return c.F / 64; }
    __device__ uint4 load_a(const Ctx&, RowA r, int kt, int lc) const { return r ? ld16(r + kt * 64 + lc * 8) : zero4(); }
    __device__ uint4 load_b(const Ctx&, RowB r, int kt, int lc) const { return r ? ld16(packed_chunk(r, kt, lc)) : zero4(); }
    template <int MB, int NB>
    __device__ __forceinline__ void epilogue(const Ctx& c, f32x16 (&acc)[MB][NB], int rb, int cb, int lane) const {
        static_for<MB>([&](auto i) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = rb + i * 32 + frag32_row(r, lane);
                // a dropped slot (destination -1) owns no output row
                const int drow = m < c.nrows ? seg.dest_of(c.seg, c.row0 + m) : -1;
                if (drow >= 0) {
                    const size_t dst = (size_t)drow * L;
                    static_for<NB>([&](auto j) {
                        const int n = c.n0 + cb + j * 32 + frag32_col(lane);
                        if (n < L) Y[dst + n] = (uint16_t)f2bf(acc[i][j][r] * c.td);
                    });
                }
            }
        });
    }
};

// =============================================================================================
// Stream (decode) problems: blocks of 16 weight rows x up to 16 tokens, K in 32-wide steps.
// Token column j reads a valid row (clamped) and is zeroed by a select when j is past the batch.
// =============================================================================================

__device__ __forceinline__ uint4 sel4(bool keep, uint4 v) { return keep ? v : zero4(); }

struct TokRow {
    const uint16_t* p;  // a valid row
    bool ok;            // column inside the batch
};

// Dense projection over token blocks of 16: mode 0 z32+z16, 1 bf16 out, 2 fp32 += out.
struct StreamProj {
    static constexpr bool kMixed = false;
    static constexpr int kSPL = 1;
    typedef uint4 WRaw;
    typedef uint4 XRaw;
    typedef uint4 XFrag;
    typedef const uint16_t* RowW;
    typedef TokRow XRow;
    const uint16_t* x;  // [T][K]
    const uint16_t* W;  // [N][K]
    int T, N, K, mode;
    float* out32;
    uint16_t* out16;
    struct Ctx { int t0, nt; };
    __device__ int num_tiles() const { return (T + 15) / 16; }
    __device__ void tile(int t, Ctx& c) const {
        c.t0 = t * 16;
        c.nt = min(16, T - c.t0);
    }
    __device__ int n_rows(const Ctx&) const { return N; }
    __device__ int k_steps(const Ctx&) const { return K / 32; }
    __device__ RowW row_w(const Ctx&, int n) const { return W + (size_t)n * K; }
    __device__ XRow x_row(const Ctx& c, int j) const { return TokRow{x + (size_t)(c.t0 + min(j, c.nt - 1)) * K, j < c.nt}; }
    template <bool>
    __device__ WRaw load_w(const Ctx&, RowW r, int, int s, int kq) const { return ld16(r + s * 32 + kq * 8); }
    template <bool>
    __device__ static uint4 wfrag(const WRaw& w, int) { return w; }
    __device__ XRaw load_x(const Ctx&, const XRow& r, int k) const { return ld16(r.p + k); }
    __device__ XFrag x_frag(const XRow& r, const XRaw& v) const { return sel4(r.ok, v); }
    __device__ static f32x4 mma(f32x4 a, uint4 w, XFrag xv) { return mfma16(w, xv, a); }
    __device__ void epilogue(const Ctx& c, int n, int j, const float* v) const {
        if (n >= N || j >= c.nt) return;
        const size_t o = (size_t)(c.t0 + j) * N + n;
        if (mode == 0) {
            out32[o] = v[0];
            out16[o] = (uint16_t)f2bf(v[0]);
        } else if (mode == 1) {
            out16[o] = (uint16_t)f2bf(v[0]);
        } else {
            out32[o] += v[0];
        }
    }
};

struct HiLo { uint4 hi, lo; };
struct F8 { float4 a, b; };

// Router logits from fp32 z: the token operand is split into hi = bf16(z), lo = bf16(z - hi),
// each multiplied by the same bf16 weights.
struct StreamRouter {
    static constexpr bool kMixed = false;
    static constexpr int kSPL = 1;
    typedef uint4 WRaw;
    typedef F8 XRaw;
    typedef HiLo XFrag;
    typedef const uint16_t* RowW;
    struct XRow { const float* p; bool ok; };
    const float* z;
    const uint16_t* W;
    const float* bias;
    int T, N, K;
    float* logits;
    struct Ctx { int t0, nt; };
    __device__ int num_tiles() const { return (T + 15) / 16; }
    __device__ void tile(int t, Ctx& c) const {
        c.t0 = t * 16;
        c.nt = min(16, T - c.t0);
    }
    __device__ int n_rows(const Ctx&) const { return N; }
    __device__ int k_steps(const Ctx&) const { return K / 32; }
    __device__ RowW row_w(const Ctx&, int n) const { return W + (size_t)n * K; }
    __device__ XRow x_row(const Ctx& c, int j) const { return XRow{z + (size_t)(c.t0 + min(j, c.nt - 1)) * K, j < c.nt}; }
    template <bool>
    __device__ WRaw load_w(const Ctx&, RowW r, int, int s, int kq) const { return ld16(r + s * 32 + kq * 8); }
    template <bool>
    __device__ static uint4 wfrag(const WRaw& w, int) { return w; }
    __device__ XRaw load_x(const Ctx&, const XRow& r, int k) const {
        return F8{*reinterpret_cast<const float4*>(r.p + k), *reinterpret_cast<const float4*>(r.p + k + 4)};
    }
    __device__ XFrag x_frag(const XRow& r, const XRaw& v) const {
        const float f[8] = {v.a.x, v.a.y, v.a.z, v.a.w, v.b.x, v.b.y, v.b.z, v.b.w};
        uint32_t h[4], l[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t h0, l0, h1, l1;
            split_hi_lo(f[2 * i], h0, l0);
            split_hi_lo(f[2 * i + 1], h1, l1);
            h[i] = h0 | (h1 << 16);
            l[i] = l0 | (l1 << 16);
        }
        return HiLo{sel4(r.ok, make_uint4(h[0], h[1], h[2], h[3])), sel4(r.ok, make_uint4(l[0], l[1], l[2], l[3]))};
    }
    __device__ static f32x4 mma(f32x4 a, uint4 w, XFrag xv) { return mfma16(w, xv.lo, mfma16(w, xv.hi, a)); }
    __device__ void epilogue(const Ctx& c, int n, int j, const float* v) const {
        if (n < N && j < c.nt) logits[(size_t)(c.t0 + j) * N + n] = v[0] + (bias ? bias[n] : 0.f);
    }
};

// ---------------------------------------------------------------------------------------------
// Expert weights for the stream kernels (packed records, see packed_row).  Q is the routed
// experts' format: 0 bf16, 1 MXFP4, 2 NVFP4.
//   bf16 records: one MFMA step per load (kSPL 1), 16 bytes per lane, 1 KB per wave.
//   4-bit records: four MFMA steps per load (kSPL 4): lane (row, kq) reads 16 bytes of
//   nibbles = the 32 values k in [128g + 32kq, +32) and their block scales; step t of the group
//   uses values 8t..8t+7 of them.  Packed 4-bit matrices are 1 KB tiles of 16 rows x 128 values
//   (unit of row j, values 32 q .. 32 q + 31 at position 16 q + j), with a scale tile per nibble
//   tile in the same unit order: MXFP4 one E8M0 byte per unit (64 bytes), NVFP4 two E4M3 bytes
//   per unit (128 bytes; the scales of its two blocks of 16).  An NVFP4 matrix also has an fp32
//   tensor scale, which multiplies the fp32 products (Mat::ts; 1 for the other formats).  In
//   4-bit kernels the (bf16) shared expert is read in the same k order: 64 bytes per lane per
//   group.
// ---------------------------------------------------------------------------------------------
struct WRaw4 { uint4 a[4]; };

template <int Q>
struct ExpertRows {
    static_assert(Q == 1 || Q == 2, "4-bit formats");
    static constexpr int kSPL = 4;
    static constexpr int kSB = Q == 1 ? 1 : 2;  // scale bytes per lane unit
    typedef WRaw4 WRaw;
    struct Mat { const uint8_t* p; const uint8_t* sc; float ts; };  // sc == null: bf16 matrix (shared expert)
    struct Row { const uint8_t* p; const uint8_t* sc; };
    __device__ static Row row(const Mat& m, int n, int K) {
        if (m.sc)
            return Row{m.p + (size_t)(n >> 4) * 8 * K + (n & 15) * 16,
                       m.sc + ((size_t)(n >> 4) * (K / 2) + (n & 15)) * kSB};
        return Row{m.p + ((size_t)(n >> 4) * 16 * K + (n & 15) * 8) * 2, nullptr};
    }
    // group g (128 values): a 4-bit lane kq holds values 32 kq .. + 32 of the group and their
    // scales; a bf16 row gives the same values as four 16-byte units (steps 4g + kq, units t)
    template <bool MXR>
    __device__ static WRaw load(const Row& r, int g, int kq) {
        WRaw w;
        if constexpr (MXR) {
            w.a[0] = ld16(r.p + g * 1024 + kq * 256);
            const uint8_t* sp = r.sc + (g * 64 + kq * 16) * kSB;
            const uint32_t sv = kSB == 1 ? (uint32_t)*sp : (uint32_t)*reinterpret_cast<const uint16_t*>(sp);
            w.a[1] = make_uint4(sv, 0, 0, 0);
            w.a[2] = w.a[3] = zero4();
        } else {
            const uint8_t* b = r.p + (size_t)(g * 4 + kq) * 1024;
#pragma unroll
            for (int t = 0; t < 4; ++t) w.a[t] = ld16(b + t * 256);
        }
        return w;
    }
    template <bool MXR>
    __device__ static uint4 frag(const WRaw& w, int t) {
        if constexpr (!MXR) {
            return w.a[t];
        } else {
            const uint32_t nib = t == 0 ? w.a[0].x : t == 1 ? w.a[0].y : t == 2 ? w.a[0].z : w.a[0].w;
            if constexpr (Q == 1) return fp4x8_to_bf16x8(nib, e8m0_to_f32(w.a[1].x));
            // steps 0, 1 hold the first block of 16 values, steps 2, 3 the second
            return fp4x8_to_bf16x8(nib, e4m3_to_f32((w.a[1].x >> (t & 2 ? 8 : 0)) & 0xFFu));
        }
    }
};

// The 4-bit rows alone, with a compact register image (16 nibble bytes and the unit's scale
// bits per lane): the small-batch kernels read bf16 rows (the shared expert) through
// ExpertRows<0> instead, so a 4-bit load needs no room for a bf16 unit.  These rows decode to
// fp16 operands (kF16; see fp4x8_to_f16x8), so their MFMAs take fp16 tokens.
template <int Q>
struct Fp4Rows {
    static constexpr int kSPL = 4;
    static constexpr bool kF16 = true;
    static constexpr int kSB = ExpertRows<Q>::kSB;
    // s: the unit's raw scale bits (MXFP4: its E8M0 byte; NVFP4: its two E4M3 bytes).  They are
    // converted where the fragments are made, not where they are loaded, so that no conversion
    // waits on a load that is still in flight.
    struct WRaw { uint4 n; uint32_t s; };
    typedef typename ExpertRows<Q>::Mat Mat;
    typedef typename ExpertRows<Q>::Row Row;
    __device__ static Row row(const Mat& m, int n, int K) { return ExpertRows<Q>::row(m, n, K); }
    template <bool>
    __device__ static WRaw load(const Row& r, int g, int kq) {
        WRaw w;
        w.n = LMOE_WLOAD(r.p + g * 1024 + kq * 256);
        const uint8_t* sp = r.sc + (g * 64 + kq * 16) * kSB;
#if LMOE_WEIGHT_NT
        w.s = Q == 1 ? (uint32_t)__builtin_nontemporal_load(sp)
                     : (uint32_t)__builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(sp));
#else
        w.s = Q == 1 ? (uint32_t)*sp : (uint32_t)*reinterpret_cast<const uint16_t*>(sp);
#endif
        return w;
    }
    template <bool>
    __device__ static uint4 frag(const WRaw& w, int t) {
        const uint32_t nib = t == 0 ? w.n.x : t == 1 ? w.n.y : t == 2 ? w.n.z : w.n.w;
        if constexpr (Q == 1) return fp4x8_to_f16x8_pow2(nib, e8m0_to_f32(w.s));
        // steps 0, 1 hold the first block of 16 values, steps 2, 3 the second
        const uint32_t s2 = e4m3x2_to_f16x2(w.s);
        return fp4x8_to_f16x8(nib, __builtin_amdgcn_perm(s2, s2, t & 2 ? 0x03020302u : 0x01000100u));
    }
};

template <>
struct ExpertRows<0> {
    static constexpr int kSPL = 1;
    static constexpr bool kF16 = false;
    typedef uint4 WRaw;
    struct Mat { const uint16_t* p; float ts; };  // packed matrix base (see packed_unit); ts = 1
    struct Row { const uint16_t* p; };            // row n: its 16-row block plus (n % 16) lane units
    __device__ static Row row(const Mat& m, int n, int K) {
        return Row{m.p + (size_t)(n >> 4) * 16 * K + (n & 15) * 8};
    }
    template <bool>
    __device__ static WRaw load(const Row& r, int s, int kq) { return LMOE_WLOAD(r.p + s * 512 + kq * 128); }
    template <bool>
    __device__ static uint4 frag(const WRaw& w, int) { return w; }
};

// Matrices of the segment a tile belongs to: the routed expert `seg` or the shared expert.
// 4-bit records: the three nibble matrices, the three scale matrices (MXFP4: [rows][K/32]
// bytes; NVFP4: [rows][K/16]), and for NVFP4 the three fp32 tensor scales.
template <int Q>
__device__ __forceinline__ void segment_mats(const void* experts, size_t rec_bytes, const uint16_t* shared, int seg,
                                             int E, int F, int Fs, int L, typename ExpertRows<Q>::Mat (&m)[3],
                                             int& Fseg, bool& mx) {
    if (seg == E) {
        Fseg = Fs;
        mx = false;
        const size_t fl = (size_t)Fs * L;
        if constexpr (Q != 0) {
            const uint8_t* b = reinterpret_cast<const uint8_t*>(shared);
            m[0] = {b, nullptr, 1.f};
            m[1] = {b + fl * 2, nullptr, 1.f};
            m[2] = {b + 2 * fl * 2, nullptr, 1.f};
        } else {
            m[0] = {shared, 1.f};
            m[1] = {shared + fl, 1.f};
            m[2] = {shared + 2 * fl, 1.f};
        }
    } else {
        Fseg = F;
        mx = Q != 0;
        const uint8_t* b = reinterpret_cast<const uint8_t*>(experts) + (size_t)seg * rec_bytes;
        const size_t fl = (size_t)F * L;
        if constexpr (Q != 0) {
            const size_t nb = fl / 2, sb = Q == 1 ? fl / 32 : fl / 16;
            float ts[3] = {1.f, 1.f, 1.f};
            if constexpr (Q == 2) {
                const float* t = reinterpret_cast<const float*>(b + 3 * nb + 3 * sb);
                ts[0] = t[0];
                ts[1] = t[1];
                ts[2] = t[2];
            }
            m[0] = {b, b + 3 * nb, ts[0]};
            m[1] = {b + nb, b + 3 * nb + sb, ts[1]};
            m[2] = {b + 2 * nb, b + 3 * nb + 2 * sb, ts[2]};
        } else {
            const uint16_t* h = reinterpret_cast<const uint16_t*>(b);
            m[0] = {h, 1.f};
            m[1] = {h + fl, 1.f};
            m[2] = {h + 2 * fl, 1.f};
        }
    }
}

// Fused gate/up (NMAT = 2) over a work list of <= 16-row tiles: H = SiLU(z gate^T) * (z up^T).
template <int Q>
struct StreamUp {
    using ER = ExpertRows<Q>;
    static constexpr bool kMixed = Q != 0;
    static constexpr int kSPL = ER::kSPL;
    typedef typename ER::WRaw WRaw;
    typedef uint4 XRaw;
    typedef uint4 XFrag;
    typedef TokRow XRow;
    struct RowW { typename ER::Row g, u; };
    SegSpace seg;
    const uint16_t* z16;
    const void* experts;
    size_t rec_bytes;
    const uint16_t* shared;
    int L, F, Fs, Hs;
    uint16_t* H;
    struct Ctx { int seg, row0, nrows, F; bool mx; typename ER::Mat m[3]; };
    __device__ int num_tiles() const { return *seg.ntiles; }
    __device__ void tile(int bx, Ctx& c) const {
        const Tile t = seg.tiles[bx];
        c.seg = t.seg;
        c.row0 = t.row0;
        c.nrows = t.nrows;
        segment_mats<Q>(experts, rec_bytes, shared, t.seg, seg.E, F, Fs, L, c.m, c.F, c.mx);
    }
    __device__ bool mx_rows(const Ctx& c) const { return c.mx; }
    __device__ int n_rows(const Ctx& c) const { return c.F; }
    __device__ int n_rows_for(int sg) const { return sg == seg.E ? Fs : F; }
    __device__ int k_steps(const Ctx&) const { return L / 32; }
    __device__ RowW row_w(const Ctx& c, int n) const { return RowW{ER::row(c.m[0], n, L), ER::row(c.m[1], n, L)}; }
    __device__ XRow x_row(const Ctx& c, int j) const {
        const int tok = seg.token_of(c.seg, c.row0 + min(j, c.nrows - 1));
        return TokRow{z16 + seg.z_off(c.seg, tok, L), j < c.nrows};
    }
    template <bool MXR>
    __device__ WRaw load_w(const Ctx&, const RowW& r, int m, int g, int kq) const {
        return ER::template load<MXR>(m == 0 ? r.g : r.u, g, kq);
    }
    template <bool MXR>
    __device__ static uint4 wfrag(const WRaw& w, int t) { return ER::template frag<MXR>(w, t); }
    __device__ XRaw load_x(const Ctx&, const XRow& r, int k) const { return ld16(r.p + k); }
    __device__ XFrag x_frag(const XRow& r, const XRaw& v) const { return sel4(r.ok, v); }
    __device__ static f32x4 mma(f32x4 a, uint4 w, XFrag xv) { return mfma16(w, xv, a); }
    __device__ void epilogue(const Ctx& c, int n, int j, const float* v) const {
        if (n < c.F && j < c.nrows)
            H[(size_t)(c.row0 + j) * Hs + n] = (uint16_t)f2bf(silu(v[0] * c.m[0].ts) * (v[1] * c.m[1].ts));
    }
};

// Down projection over a work list: Y[dest(p)][n] = H[p] . down[n].
template <int Q>
struct StreamDown {
    using ER = ExpertRows<Q>;
    static constexpr bool kMixed = Q != 0;
    static constexpr int kSPL = ER::kSPL;
    typedef typename ER::WRaw WRaw;
    typedef uint4 XRaw;
    typedef uint4 XFrag;
    typedef TokRow XRow;
    typedef typename ER::Row RowW;
    SegSpace seg;
    const uint16_t* H;
    const void* experts;
    size_t rec_bytes;
    const uint16_t* shared;
    int L, F, Fs, Hs;
    uint16_t* Y;  // [R][L] bf16
    struct Ctx { int seg, row0, nrows, F; bool mx; typename ER::Mat m[3]; };
    __device__ int num_tiles() const { return *seg.ntiles; }
    __device__ void tile(int bx, Ctx& c) const {
        const Tile t = seg.tiles[bx];
        c.seg = t.seg;
        c.row0 = t.row0;
        c.nrows = t.nrows;
        segment_mats<Q>(experts, rec_bytes, shared, t.seg, seg.E, F, Fs, L, c.m, c.F, c.mx);
    }
    __device__ bool mx_rows(const Ctx& c) const { return c.mx; }
    __device__ int n_rows(const Ctx&) const { return L; }
    __device__ int k_steps(const Ctx& c) const { return c.F / 32; }
    __device__ RowW row_w(const Ctx& c, int n) const { return ER::row(c.m[2], n, c.F); }
    __device__ XRow x_row(const Ctx& c, int j) const {
        return TokRow{H + (size_t)(c.row0 + min(j, c.nrows - 1)) * Hs, j < c.nrows};
    }
    template <bool MXR>
    __device__ WRaw load_w(const Ctx&, const RowW& r, int, int g, int kq) const { return ER::template load<MXR>(r, g, kq); }
    template <bool MXR>
    __device__ static uint4 wfrag(const WRaw& w, int t) { return ER::template frag<MXR>(w, t); }
    __device__ XRaw load_x(const Ctx&, const XRow& r, int k) const { return ld16(r.p + k); }
    __device__ XFrag x_frag(const XRow& r, const XRaw& v) const { return sel4(r.ok, v); }
    __device__ static f32x4 mma(f32x4 a, uint4 w, XFrag xv) { return mfma16(w, xv, a); }
    __device__ void epilogue(const Ctx& c, int n, int j, const float* v) const {
        if (n >= L || j >= c.nrows) return;
        const int drow = seg.dest_of(c.seg, c.row0 + j);
        if (drow >= 0) Y[(size_t)drow * L + n] = (uint16_t)f2bf(v[0] * c.m[2].ts);
    }
};

}  // namespace lmoe

// =============================================================================================
// Pipelined (global -> LDS) problems: the tile problems' contexts and epilogues, plus the
// per-lane source of each 1 KB copy of a stage (row-major operands: 8 rows per copy; packed
// expert weights: one 16 x 32 tile per copy).  Rows outside the problem are clamped to a valid
// row.
// =============================================================================================
#include "gemm_pipe.hpp"

namespace lmoe {

template <class S>
struct PipeProj : TileProj<S> {
    using B = TileProj<S>;
    static constexpr bool kAPacked = false, kBPacked = false, kLdsStore = true;
    __device__ int m_tiles() const { return (B::M + S::kBM - 1) / S::kBM; }
    __device__ int valid_rows(const typename B::Ctx& c) const { return min(S::kBM, B::M - c.m0); }
    __device__ int k_stages(const typename B::Ctx&) const { return B::K / S::kBK; }
    __device__ const uint8_t* a_base(const typename B::Ctx& c) const {
        return reinterpret_cast<const uint8_t*>(B::x + (size_t)c.m0 * B::K);
    }
    __device__ const uint8_t* b_base(const typename B::Ctx& c) const {
        return reinterpret_cast<const uint8_t*>(B::W + (size_t)c.n0 * B::K);
    }
    __device__ uint32_t src_a(const typename B::Ctx& c, int i, int lane) const {
        const int r = min(rowmajor_row<S::kU>(i, lane), B::M - 1 - c.m0);
        return rowmajor_off<S::kU>((uint32_t)r * B::K * 2, i, lane);
    }
    __device__ uint32_t src_b(const typename B::Ctx& c, int i, int lane) const {
        const int r = min(rowmajor_row<S::kU>(i, lane), B::N - 1 - c.n0);
        return rowmajor_off<S::kU>((uint32_t)r * B::K * 2, i, lane);
    }
    struct Prep {};
    template <int MB>
    __device__ Prep prep(const typename B::Ctx&, int, int) const { return {}; }
    // The outputs of TileProj's modes from the transposed accumulators: a lane holds one row of
    // each 32-row block and four consecutive n per register group, so modes 0-2 store 4 values
    // at a time (N is a multiple of 64 and every tensor 16-byte aligned); mode 3 interleaves
    // the router halves (n = 2e + h) and stores them one by one.
    template <int MD, int MB, int NB>
    __device__ __forceinline__ void store_mode(const typename B::Ctx& c, f32x16 (&acc)[MB][NB], int rb, int cb,
                                               int lane) const {
        const int h4 = 4 * (lane >> 5);
        static_for<MB>([&](auto i) {
            const int m = c.m0 + rb + i * 32 + (lane & 31);
            if (m < B::M) {
                static_for<NB>([&](auto j) {
#pragma unroll
                    for (int r4 = 0; r4 < 4; ++r4) {
                        const int n = c.n0 + cb + j * 32 + 8 * r4 + h4;
                        const f32x16& a = acc[i][j];
                        const float v[4] = {a[4 * r4], a[4 * r4 + 1], a[4 * r4 + 2], a[4 * r4 + 3]};
                        const size_t o = (size_t)m * B::N + n;
                        if constexpr (MD == 3) {
#pragma unroll
                            for (int t = 0; t < 4; ++t) {
                                const int nt = n + t, e = nt >> 1, h = nt & 1;
                                if (nt < B::N)
                                    B::out32[((size_t)h * B::M + m) * (B::N >> 1) + e] =
                                        h == 0 && B::bias ? v[t] + B::bias[e] : v[t];
                            }
                        } else if (n < B::N) {
                            if constexpr (MD == 0) {
                                uint32_t hi[4], lo[4];
#pragma unroll
                                for (int t = 0; t < 4; ++t) split_hi_lo(v[t], hi[t], lo[t]);
                                if (B::out32)
                                    *reinterpret_cast<float4*>(B::out32 + o) = make_float4(v[0], v[1], v[2], v[3]);
                                *reinterpret_cast<uint2*>(B::out16 + o) = make_uint2(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16));
                                if (B::out16lo)
                                    *reinterpret_cast<uint2*>(B::out16lo + o) =
                                        make_uint2(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16));
                            } else if constexpr (MD == 1) {
                                *reinterpret_cast<uint2*>(B::out16 + o) =
                                    make_uint2(pack_bf2_rn(v[0], v[1]), pack_bf2_rn(v[2], v[3]));
                            } else {
                                float4* q = reinterpret_cast<float4*>(B::out32 + o);
                                float4 r = *q;
                                r.x += v[0];
                                r.y += v[1];
                                r.z += v[2];
                                r.w += v[3];
                                *q = r;
                            }
                        }
                    }
                });
            }
        });
    }
    // bf16 outputs staged through LDS (staged_store_bf16): mode 1, and the high half of mode 0
    // without the fp32 output; the other forms store from the accumulators once the next tile's
    // first stages are issued.
    template <class SS, int MB, int NB, class F>
    __device__ __forceinline__ void store_lds(const typename B::Ctx& c, f32x16 (&acc)[MB][NB], Prep p, int rb, int cb,
                                              int lane, int wave, uint4* st0, uint4* st1, uint4* st2,
                                              F&& issue_next) const {
        static_assert(SS::kBN == 256, "256-column tiles");
        auto chunk_of = [&](int j, int r4) { return (cb + j * 32) / 8 + r4; };
        auto row_of = [&](int r) { return c.m0 + r < B::M ? c.m0 + r : -1; };
        if (B::mode == 1) {
            staged_store_bf16<SS, 32, NB, true, MB, NB>(
                lane, wave, st0, st1, st2,
                [&](int i, int j, int r4) {
                    const f32x16& v = acc[i][j];
                    return make_uint2(pack_bf2_rn(v[4 * r4], v[4 * r4 + 1]), pack_bf2_rn(v[4 * r4 + 2], v[4 * r4 + 3]));
                },
                chunk_of, row_of, B::out16, (size_t)B::N, c.n0, B::N, issue_next);
        } else if (B::mode == 0 && !B::out32) {
            // the low halves straight from the accumulators (8 bytes a lane), then the high halves
            // staged
            if (B::out16lo) {
                const int h4 = 4 * (lane >> 5);
                static_for<MB>([&](auto i) {
                    const int m = c.m0 + rb + i * 32 + (lane & 31);
                    if (m < B::M)
                        static_for<NB>([&](auto j) {
#pragma unroll
                            for (int r4 = 0; r4 < 4; ++r4) {
                                const int n = c.n0 + cb + j * 32 + 8 * r4 + h4;
                                if (n < B::N) {
                                    uint32_t hi[4], lo[4];
#pragma unroll
                                    for (int t = 0; t < 4; ++t) split_hi_lo(acc[i][j][4 * r4 + t], hi[t], lo[t]);
                                    *reinterpret_cast<uint2*>(B::out16lo + (size_t)m * B::N + n) =
                                        make_uint2(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16));
                                }
                            }
                        });
                });
            }
            staged_store_bf16<SS, 32, NB, true, MB, NB>(
                lane, wave, st0, st1, st2,
                [&](int i, int j, int r4) {
                    const f32x16& v = acc[i][j];
                    uint32_t hi[4];
#pragma unroll
                    for (int t = 0; t < 4; ++t) hi[t] = f2bf(v[4 * r4 + t]);
                    return make_uint2(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16));
                },
                chunk_of, row_of, B::out16, (size_t)B::N, c.n0, B::N, issue_next);
        } else {
            issue_next();
            store<MB, NB>(c, acc, p, rb, cb, lane);
        }
    }
    template <int MB, int NB>
    __device__ __forceinline__ void store(const typename B::Ctx& c, f32x16 (&acc)[MB][NB], Prep, int rb, int cb,
                                          int lane) const {
        if (B::mode == 0)
            store_mode<0>(c, acc, rb, cb, lane);
        else if (B::mode == 1)
            store_mode<1>(c, acc, rb, cb, lane);
        else if (B::mode == 2)
            store_mode<2>(c, acc, rb, cb, lane);
        else
            store_mode<3>(c, acc, rb, cb, lane);
    }
};

// Router logits of a batch from the two bf16 halves of z (hi = bf16(z), lo = bf16(z - hi)):
// out[h][m][n] = z_h[m] . W[n] (+ bias[n] for h = 0); the top-k adds the two halves.  The halves
// are two M ranges of one launch (tiles [0, mt) multiply hi, [mt, 2 mt) lo).
template <class S>
struct PipeRouter {
    const uint16_t* zhi;  // [M][K] bf16
    const uint16_t* zlo;  // [M][K] bf16
    const uint16_t* W;    // [N][K] bf16 router rows
    const float* bias;    // [N] or null
    int M, N, K;
    float* out;  // [2][M][N]
    static constexpr bool kAPacked = false, kBPacked = false, kLdsStore = false;
    struct Ctx { int m0, n0, h; };
    __device__ int mt() const { return (M + S::kBM - 1) / S::kBM; }
    __device__ int m_tiles() const { return 2 * mt(); }
    __device__ bool tile(int bx, int by, Ctx& c) const {
        const int t = mt();
        c.h = bx >= t ? 1 : 0;
        c.m0 = (bx - c.h * t) * S::kBM;
        c.n0 = by * S::kBN;
        return c.m0 < M && c.n0 < N;
    }
    __device__ int valid_rows(const Ctx& c) const { return min(S::kBM, M - c.m0); }
    __device__ int k_stages(const Ctx&) const { return K / S::kBK; }
    __device__ const uint8_t* a_base(const Ctx& c) const {
        return reinterpret_cast<const uint8_t*>((c.h ? zlo : zhi) + (size_t)c.m0 * K);
    }
    __device__ const uint8_t* b_base(const Ctx& c) const { return reinterpret_cast<const uint8_t*>(W + (size_t)c.n0 * K); }
    __device__ uint32_t src_a(const Ctx& c, int i, int lane) const {
        const int r = min(rowmajor_row<S::kU>(i, lane), M - 1 - c.m0);
        return rowmajor_off<S::kU>((uint32_t)r * K * 2, i, lane);
    }
    __device__ uint32_t src_b(const Ctx& c, int i, int lane) const {
        const int r = min(rowmajor_row<S::kU>(i, lane), N - 1 - c.n0);
        return rowmajor_off<S::kU>((uint32_t)r * K * 2, i, lane);
    }
    struct Prep {};
    template <int MB>
    __device__ Prep prep(const Ctx&, int, int) const { return {}; }
    // four consecutive n of one row per lane and register group (16-byte stores when N is a
    // multiple of 4, else one by one)
    template <int MB, int NB>
    __device__ __forceinline__ void store(const Ctx& c, f32x16 (&acc)[MB][NB], Prep, int rb, int cb, int lane) const {
        const int h4 = 4 * (lane >> 5);
        const bool vec = (N & 3) == 0;
        const float* bz = c.h == 0 ? bias : nullptr;
        static_for<MB>([&](auto i) {
            const int m = c.m0 + rb + i * 32 + (lane & 31);
            if (m < M) {
                float* orow = out + ((size_t)c.h * M + m) * N;
                static_for<NB>([&](auto j) {
#pragma unroll
                    for (int r4 = 0; r4 < 4; ++r4) {
                        const int n = c.n0 + cb + j * 32 + 8 * r4 + h4;
                        float v[4];
#pragma unroll
                        for (int t = 0; t < 4; ++t) v[t] = acc[i][j][4 * r4 + t] + (bz && n + t < N ? bz[n + t] : 0.f);
                        if (vec) {
                            if (n < N) *reinterpret_cast<float4*>(orow + n) = make_float4(v[0], v[1], v[2], v[3]);
                        } else {
#pragma unroll
                            for (int t = 0; t < 4; ++t)
                                if (n + t < N) orow[n + t] = v[t];
                        }
                    }
                });
            }
        });
    }
};

template <class S>
struct PipeUp : TileUp<S> {
    using B = TileUp<S>;
    static constexpr bool kAPacked = false, kBPacked = true, kLdsStore = true;
    __device__ int m_tiles() const { return B::seg.count(); }
    __device__ int valid_rows(const typename B::Ctx& c) const { return c.nrows; }
    __device__ int k_stages(const typename B::Ctx&) const { return B::L / S::kBK; }
    __device__ const uint8_t* a_base(const typename B::Ctx&) const { return reinterpret_cast<const uint8_t*>(B::z16); }
    __device__ const uint8_t* b_base(const typename B::Ctx& c) const { return reinterpret_cast<const uint8_t*>(c.g); }
    // gathered token rows: byte offsets into z16 stay below 2^32 (T * zp * 2 < 2^32 is checked
    // on the host)
    __device__ uint32_t src_a(const typename B::Ctx& c, int i, int lane) const {
        const int r = min(rowmajor_row<S::kU>(i, lane), c.nrows - 1);
        return rowmajor_off<S::kU>((uint32_t)(B::seg.z_off(c.seg, B::seg.token_of(c.seg, c.row0 + r), B::L) * 2), i,
                                   lane);
    }
    __device__ uint32_t src_b(const typename B::Ctx& c, int i, int lane) const {
        const int r = packed_block<S::kU>(i) * 16;  // first B-tile row of this copy (16 rows: one matrix, one f block)
        const int wc = r / S::kWN, rr = r % S::kWN;
        const int f = c.f0 + wc * B::kHalf + rr % B::kHalf;
        const int nb = min(f, c.F - 16) >> 4;
        const uint32_t mat = rr >= B::kHalf ? (uint32_t)c.F * B::L * 2 : 0u;  // up follows gate
        return mat + packed_off<S::kU>(nb, i, B::L, lane);
    }
    struct Prep {};
    template <int MB>
    __device__ Prep prep(const typename B::Ctx&, int, int) const { return {}; }
    // H[row][f] = bf16(silu(gate * tg) * (up * tu)), staged through LDS (staged_store_bf16): a
    // 256-column tile holds 128 gate and 128 up columns, so its H tile is 128 columns (16 chunks)
    // wide, the gate blocks j < NB / 2 of wave column wn giving H columns wn * kHalf + 32 j ..
    template <class SS, int MB, int NB, class F>
    __device__ __forceinline__ void store_lds(const typename B::Ctx& c, f32x16 (&acc)[MB][NB], Prep, int rb, int cb,
                                              int lane, int wave, uint4* st0, uint4* st1, uint4* st2,
                                              F&& issue_next) const {
        static_assert(NB % 2 == 0 && NB * 16 == B::kHalf && SS::kBN == 256, "gate blocks then up blocks per wave column");
        const int wn = cb / SS::kWN;
        staged_store_bf16<SS, 16, NB / 2, true, MB, NB>(
            lane, wave, st0, st1, st2,
            [&](int i, int j, int r4) {
                float h[4];
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    h[t] = silu(acc[i][j][4 * r4 + t] * c.tg) * (acc[i][j + NB / 2][4 * r4 + t] * c.tu);
                return make_uint2(pack_bf2_rn(h[0], h[1]), pack_bf2_rn(h[2], h[3]));
            },
            [&](int j, int r4) { return (wn * B::kHalf + j * 32) / 8 + r4; },
            [&](int r) { return r < c.nrows ? c.row0 + r : -1; }, B::H, (size_t)B::Hs, c.f0, c.F, issue_next);
    }
};

template <class S>
struct PipeDown : TileDown<S> {
    using B = TileDown<S>;
    static constexpr bool kAPacked = false, kBPacked = true, kLdsStore = true;
    __device__ int m_tiles() const { return B::seg.count(); }
    __device__ int valid_rows(const typename B::Ctx& c) const { return c.nrows; }
    __device__ int k_stages(const typename B::Ctx& c) const { return c.F / S::kBK; }
    __device__ const uint8_t* a_base(const typename B::Ctx& c) const {
        return reinterpret_cast<const uint8_t*>(B::H + (size_t)c.row0 * B::Hs);
    }
    __device__ const uint8_t* b_base(const typename B::Ctx& c) const { return reinterpret_cast<const uint8_t*>(c.d); }
    __device__ uint32_t src_a(const typename B::Ctx& c, int i, int lane) const {
        const int r = min(rowmajor_row<S::kU>(i, lane), c.nrows - 1);
        return rowmajor_off<S::kU>((uint32_t)r * B::Hs * 2, i, lane);
    }
    __device__ uint32_t src_b(const typename B::Ctx& c, int i, int lane) const {
        const int nb = min(c.n0 + packed_block<S::kU>(i) * 16, B::L - 16) >> 4;
        return packed_off<S::kU>(nb, i, c.F, lane);
    }
    // Destination row of every row of the tile (-1: none) in LDS, written before the barrier that
    // precedes the store (the store reads the rows of other waves).
    __device__ static int* prep_rows() {
        __shared__ int rows[S::kBM];
        return rows;
    }
    struct Prep {};
    template <int MB>
    __device__ __forceinline__ Prep prep(const typename B::Ctx& c, int, int) const {
        int* rows = prep_rows();
        for (int m = threadIdx.x; m < S::kBM; m += S::kThreads)
            rows[m] = m < c.nrows ? B::seg.dest_of(c.seg, c.row0 + m) : -1;
        return {};
    }
    // Y[dest][n] = bf16(acc * td), staged through LDS (staged_store_bf16: whole row segments per
    // store instruction).
    template <class SS, int MB, int NB, class F>
    __device__ __forceinline__ void store_lds(const typename B::Ctx& c, f32x16 (&acc)[MB][NB], Prep, int rb, int cb,
                                              int lane, int wave, uint4* st0, uint4* st1, uint4* st2,
                                              F&& issue_next) const {
        static_assert(SS::kBN == 256, "256-column tiles");
        const int* rows = prep_rows();
        staged_store_bf16<SS, 32, NB, true, MB, NB>(
            lane, wave, st0, st1, st2,
            [&](int i, int j, int r4) {
                const f32x16& v = acc[i][j];
                return make_uint2(pack_bf2_rn(v[4 * r4] * c.td, v[4 * r4 + 1] * c.td),
                                  pack_bf2_rn(v[4 * r4 + 2] * c.td, v[4 * r4 + 3] * c.td));
            },
            [&](int j, int r4) { return (cb + j * 32) / 8 + r4; }, [&](int r) { return rows[r]; }, B::Y, (size_t)B::L,
            c.n0, B::L, issue_next);
    }
};

}  // namespace lmoe
