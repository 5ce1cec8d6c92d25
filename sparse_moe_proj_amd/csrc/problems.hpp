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
    // a dropped slot (perm = -1) maps to token 0: its rows are computed but never stored
    __device__ __forceinline__ int token_of(int seg, int p) const { return seg == E ? p - T * k : max(perm[p], 0) / k; }
    __device__ __forceinline__ int dest_of(int seg, int p) const { return seg == E ? p : perm[p]; }
};

// =============================================================================================
// Tile (prefill) problems: 128x128 tiles, 2x2 waves of 64x64.
// =============================================================================================
using Tile128 = TileShape<128, 128, 2, 2>;

// Dense projection C[t][n] = x[t] . W[n]; mode 0: z32 + z16 (D), 1: bf16 y (U), 2: y += (U, fp32 residual)
struct TileProj {
    const uint16_t* x;  // [M][K] bf16
    const uint16_t* W;  // [N][K] bf16
    int M, N, K, mode;
    float* out32;
    uint16_t* out16;
    struct Ctx { int m0, n0; };
    typedef const uint16_t* RowA;
    typedef const uint16_t* RowB;
    __device__ bool tile(int bx, int by, Ctx& c) const {
        c.m0 = bx * Tile128::kBM;
        c.n0 = by * Tile128::kBN;
        return c.m0 < M && c.n0 < N;
    }
    __device__ RowA row_a(const Ctx& c, int r) const { return c.m0 + r < M ? x + (size_t)(c.m0 + r) * K : nullptr; }
    __device__ RowB row_b(const Ctx& c, int r) const { return c.n0 + r < N ? W + (size_t)(c.n0 + r) * K : nullptr; }
    __device__ int k_tiles(const Ctx&) const { return K / 64; }
    __device__ uint4 load_a(const Ctx&, RowA r, int kt, int lc) const { return r ? ld16(r + kt * 64 + lc * 8) : zero4(); }
    __device__ uint4 load_b(const Ctx&, RowB r, int kt, int lc) const { return r ? ld16(r + kt * 64 + lc * 8) : zero4(); }
    template <int MB, int NB>
    __device__ void epilogue(const Ctx& c, f32x16 (&acc)[MB][NB], int rb, int cb, int lane) const {
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = c.m0 + rb + i * 32 + frag32_row(r, lane);
                    const int n = c.n0 + cb + j * 32 + frag32_col(lane);
                    if (m < M && n < N) {
                        const float v = acc[i][j][r];
                        const size_t o = (size_t)m * N + n;
                        if (mode == 0) {
                            out32[o] = v;
                            out16[o] = (uint16_t)f2bf(v);
                        } else if (mode == 1) {
                            out16[o] = (uint16_t)f2bf(v);
                        } else {
                            out32[o] += v;
                        }
                    }
                }
    }
};

// Router logits from fp32 z: K doubled, first half multiplies hi(z), second half lo(z), same Wr.
struct TileRouter {
    const float* z;      // [M][K] fp32
    const uint16_t* W;   // [E][K] bf16
    const float* bias;   // [E] or null
    int M, N, K;
    float* logits;       // [M][N]
    struct Ctx { int m0, n0; };
    typedef const float* RowA;
    typedef const uint16_t* RowB;
    __device__ bool tile(int bx, int by, Ctx& c) const {
        c.m0 = bx * Tile128::kBM;
        c.n0 = by * Tile128::kBN;
        return c.m0 < M && c.n0 < N;
    }
    __device__ RowA row_a(const Ctx& c, int r) const { return c.m0 + r < M ? z + (size_t)(c.m0 + r) * K : nullptr; }
    __device__ RowB row_b(const Ctx& c, int r) const { return c.n0 + r < N ? W + (size_t)(c.n0 + r) * K : nullptr; }
    __device__ int k_tiles(const Ctx&) const { return 2 * (K / 64); }
    __device__ uint4 load_a(const Ctx&, RowA r, int kt, int lc) const {
        if (!r) return zero4();
        const int h = K / 64;
        const bool lo = kt >= h;
        return f32x8_to_bf16_part(r + (lo ? kt - h : kt) * 64 + lc * 8, lo);
    }
    __device__ uint4 load_b(const Ctx&, RowB r, int kt, int lc) const {
        if (!r) return zero4();
        const int h = K / 64;
        return ld16(r + (kt >= h ? kt - h : kt) * 64 + lc * 8);
    }
    template <int MB, int NB>
    __device__ void epilogue(const Ctx& c, f32x16 (&acc)[MB][NB], int rb, int cb, int lane) const {
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = c.m0 + rb + i * 32 + frag32_row(r, lane);
                    const int n = c.n0 + cb + j * 32 + frag32_col(lane);
                    if (m < M && n < N) logits[(size_t)m * N + n] = acc[i][j][r] + (bias ? bias[n] : 0.f);
                }
    }
};

// Fused SwiGLU gate/up over a work list.  The B tile's 128 rows are, for each of the two
// wave columns, 32 gate rows followed by the same 32 up rows, so every lane ends with g and u
// of the same (row, f) in acc[i][0] / acc[i][1] and applies SiLU(g) * u in registers.
struct TileUp {
    SegSpace seg;
    const uint16_t* z16;      // [T][L]
    const uint16_t* experts;  // E records
    const uint16_t* shared;   // record or null
    size_t rec;               // elements per routed record
    int L, F, Fs, Hs;
    uint16_t* H;              // [R][Hs]
    struct Ctx { int seg, row0, nrows, F, f0; const uint16_t* g; const uint16_t* u; };
    typedef const uint16_t* RowA;
    typedef const uint16_t* RowB;
    __device__ bool tile(int bx, int by, Ctx& c) const {
        if (bx >= *seg.ntiles) return false;
        const Tile t = seg.tiles[bx];
        c.seg = t.seg;
        c.row0 = t.row0;
        c.nrows = t.nrows;
        if (t.seg == seg.E) {
            c.F = Fs;
            c.g = shared;
        } else {
            c.F = F;
            c.g = experts + (size_t)t.seg * rec;
        }
        c.u = c.g + (size_t)c.F * L;
        c.f0 = by * 64;
        return c.f0 < c.F;
    }
    __device__ RowA row_a(const Ctx& c, int r) const {
        if (r >= c.nrows) return nullptr;
        return z16 + (size_t)seg.token_of(c.seg, c.row0 + r) * L;
    }
    __device__ RowB row_b(const Ctx& c, int r) const {
        const int f = c.f0 + (r >> 6) * 32 + (r & 31);
        if (f >= c.F) return nullptr;
        return ((r >> 5) & 1 ? c.u : c.g) + (size_t)f * L;
    }
    __device__ int k_tiles(const Ctx&) const { return L / 64; }
    __device__ uint4 load_a(const Ctx&, RowA r, int kt, int lc) const { return r ? ld16(r + kt * 64 + lc * 8) : zero4(); }
    __device__ uint4 load_b(const Ctx&, RowB r, int kt, int lc) const { return r ? ld16(r + kt * 64 + lc * 8) : zero4(); }
    template <int MB, int NB>
    __device__ void epilogue(const Ctx& c, f32x16 (&acc)[MB][NB], int rb, int cb, int lane) const {
        static_assert(NB == 2, "gate block + up block per wave column");
        const int f = c.f0 + (cb >> 6) * 32 + frag32_col(lane);
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = rb + i * 32 + frag32_row(r, lane);
                if (m < c.nrows && f < c.F)
                    H[(size_t)(c.row0 + m) * Hs + f] = (uint16_t)f2bf(silu(acc[i][0][r]) * acc[i][1][r]);
            }
    }
};

// Down projection over a work list: Y[dest(p)][n] = H[p] . down[n].
struct TileDown {
    SegSpace seg;
    const uint16_t* H;
    const uint16_t* experts;
    const uint16_t* shared;
    size_t rec;
    int L, F, Fs, Hs;
    float* Y;  // [R][L]
    struct Ctx { int seg, row0, nrows, F, n0; const uint16_t* d; };
    typedef const uint16_t* RowA;
    typedef const uint16_t* RowB;
    __device__ bool tile(int bx, int by, Ctx& c) const {
        if (bx >= *seg.ntiles) return false;
        const Tile t = seg.tiles[bx];
        c.seg = t.seg;
        c.row0 = t.row0;
        c.nrows = t.nrows;
        if (t.seg == seg.E) {
            c.F = Fs;
            c.d = shared + 2 * (size_t)Fs * L;
        } else {
            c.F = F;
            c.d = experts + (size_t)t.seg * rec + 2 * (size_t)F * L;
        }
        c.n0 = by * Tile128::kBN;
        return c.n0 < L;
    }
    __device__ RowA row_a(const Ctx& c, int r) const { return r < c.nrows ? H + (size_t)(c.row0 + r) * Hs : nullptr; }
    __device__ RowB row_b(const Ctx& c, int r) const { return c.n0 + r < L ? c.d + (size_t)(c.n0 + r) * c.F : nullptr; }
    __device__ int k_tiles(const Ctx& c) const { return c.F / 64; }
    __device__ uint4 load_a(const Ctx&, RowA r, int kt, int lc) const { return r ? ld16(r + kt * 64 + lc * 8) : zero4(); }
    __device__ uint4 load_b(const Ctx&, RowB r, int kt, int lc) const { return r ? ld16(r + kt * 64 + lc * 8) : zero4(); }
    template <int MB, int NB>
    __device__ void epilogue(const Ctx& c, f32x16 (&acc)[MB][NB], int rb, int cb, int lane) const {
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = rb + i * 32 + frag32_row(r, lane);
                if (m >= c.nrows) continue;
                const int drow = seg.dest_of(c.seg, c.row0 + m);
                if (drow < 0) continue;  // a dropped slot owns no output row
                const size_t dst = (size_t)drow * L;
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    const int n = c.n0 + cb + j * 32 + frag32_col(lane);
                    if (n < L) Y[dst + n] = acc[i][j][r];
                }
            }
    }
};

// =============================================================================================
// Stream (decode) problems: 16 weight rows x up to 16 tokens, K in 32-wide steps.
// =============================================================================================

// Dense projection over token blocks of 16: mode 0 z32+z16, 1 bf16 out, 2 fp32 += out.
struct StreamProj {
    const uint16_t* x;  // [T][K]
    const uint16_t* W;  // [N][K]
    int T, N, K, mode;
    float* out32;
    uint16_t* out16;
    struct Ctx { int t0, nt; };
    typedef const uint16_t* RowW;
    typedef const uint16_t* RowX;
    typedef uint4 XFrag;
    __device__ bool tile(int by, Ctx& c) const {
        c.t0 = by * 16;
        c.nt = min(16, T - c.t0);
        return c.nt > 0;
    }
    __device__ int n_rows(const Ctx&) const { return N; }
    __device__ int k_steps(const Ctx&) const { return K / 32; }
    __device__ RowW row_w(const Ctx&, int n) const { return n < N ? W + (size_t)n * K : nullptr; }
    __device__ RowX row_x(const Ctx& c, int j) const { return j < c.nt ? x + (size_t)(c.t0 + j) * K : nullptr; }
    __device__ uint4 load_w(const Ctx&, RowW r, int, int s, int kq) const { return r ? ld16(r + s * 32 + kq * 8) : zero4(); }
    __device__ XFrag load_x(const Ctx&, RowX r, int s, int kq) const { return r ? ld16(r + s * 32 + kq * 8) : zero4(); }
    __device__ static f32x4 mma(f32x4 a, uint4 w, XFrag x) { return mfma16(w, x, a); }
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

// Router logits from fp32 z (hi/lo bf16 split of the token operand).
struct StreamRouter {
    const float* z;
    const uint16_t* W;
    const float* bias;
    int T, N, K;
    float* logits;
    struct Ctx { int t0, nt; };
    typedef const uint16_t* RowW;
    typedef const float* RowX;
    typedef HiLo XFrag;
    __device__ bool tile(int by, Ctx& c) const {
        c.t0 = by * 16;
        c.nt = min(16, T - c.t0);
        return c.nt > 0;
    }
    __device__ int n_rows(const Ctx&) const { return N; }
    __device__ int k_steps(const Ctx&) const { return K / 32; }
    __device__ RowW row_w(const Ctx&, int n) const { return n < N ? W + (size_t)n * K : nullptr; }
    __device__ RowX row_x(const Ctx& c, int j) const { return j < c.nt ? z + (size_t)(c.t0 + j) * K : nullptr; }
    __device__ uint4 load_w(const Ctx&, RowW r, int, int s, int kq) const { return r ? ld16(r + s * 32 + kq * 8) : zero4(); }
    __device__ XFrag load_x(const Ctx&, RowX r, int s, int kq) const {
        HiLo h;
        if (!r) {
            h.hi = h.lo = zero4();
        } else {
            h.hi = f32x8_to_bf16_part(r + s * 32 + kq * 8, false);
            h.lo = f32x8_to_bf16_part(r + s * 32 + kq * 8, true);
        }
        return h;
    }
    __device__ static f32x4 mma(f32x4 a, uint4 w, XFrag x) { return mfma16(w, x.lo, mfma16(w, x.hi, a)); }
    __device__ void epilogue(const Ctx& c, int n, int j, const float* v) const {
        if (n < N && j < c.nt) logits[(size_t)(c.t0 + j) * N + n] = v[0] + (bias ? bias[n] : 0.f);
    }
};

// Weight-row addressing for one expert matrix in bf16 or MXFP4.
template <bool MX>
struct WRow;
template <>
struct WRow<false> {
    const uint16_t* p;
    __device__ uint4 load(int s, int kq) const { return p ? ld16(p + s * 32 + kq * 8) : zero4(); }
};
template <>
struct WRow<true> {
    const uint8_t* nib;  // row's packed nibbles (K/2 bytes)
    const uint8_t* sc;   // row's scale bytes (K/32)
    __device__ uint4 load(int s, int kq) const {
        if (!nib) return zero4();
        const uint32_t w = *reinterpret_cast<const uint32_t*>(nib + s * 16 + kq * 4);
        return mxfp4_to_bf16x8(w, sc[s]);
    }
};

// Locations of one routed expert's three matrices.
template <bool MX>
struct ExpertMats;
template <>
struct ExpertMats<false> {
    const uint16_t *g, *u, *d;
    __device__ static ExpertMats make(const void* base, size_t rec_bytes, int e, int F, int L) {
        const uint16_t* b = reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(base) + (size_t)e * rec_bytes);
        return ExpertMats{b, b + (size_t)F * L, b + 2 * (size_t)F * L};
    }
    __device__ WRow<false> gate(int n, int L) const { return WRow<false>{g + (size_t)n * L}; }
    __device__ WRow<false> up(int n, int L) const { return WRow<false>{u + (size_t)n * L}; }
    __device__ WRow<false> down(int n, int F) const { return WRow<false>{d + (size_t)n * F}; }
};
template <>
struct ExpertMats<true> {
    const uint8_t *g, *u, *d, *gs, *us, *ds;
    __device__ static ExpertMats make(const void* base, size_t rec_bytes, int e, int F, int L) {
        const uint8_t* b = reinterpret_cast<const uint8_t*>(base) + (size_t)e * rec_bytes;
        const size_t nb = (size_t)F * L / 2, sb = (size_t)F * L / 32;
        return ExpertMats{b, b + nb, b + 2 * nb, b + 3 * nb, b + 3 * nb + sb, b + 3 * nb + 2 * sb};
    }
    __device__ WRow<true> gate(int n, int L) const { return WRow<true>{g + (size_t)n * (L / 2), gs + (size_t)n * (L / 32)}; }
    __device__ WRow<true> up(int n, int L) const { return WRow<true>{u + (size_t)n * (L / 2), us + (size_t)n * (L / 32)}; }
    __device__ WRow<true> down(int n, int F) const { return WRow<true>{d + (size_t)n * (F / 2), ds + (size_t)n * (F / 32)}; }
};

// Fused gate/up (NMAT = 2) over a work list of <= 16-row tiles; MX: routed experts in MXFP4
// (the shared expert is always bf16).
template <bool MX>
struct StreamUp {
    SegSpace seg;
    const uint16_t* z16;
    const void* experts;
    size_t rec_bytes;
    const uint16_t* shared;
    int L, F, Fs, Hs;
    uint16_t* H;
    struct Ctx { int seg, row0, nrows, F; ExpertMats<MX> em; ExpertMats<false> sm; };
    struct RowW { WRow<MX> g, u; WRow<false> sg, su; bool sh; };
    typedef const uint16_t* RowX;
    typedef uint4 XFrag;
    __device__ bool tile(int by, Ctx& c) const {
        if (by >= *seg.ntiles) return false;
        const Tile t = seg.tiles[by];
        c.seg = t.seg;
        c.row0 = t.row0;
        c.nrows = t.nrows;
        if (t.seg == seg.E) {
            c.F = Fs;
            c.sm = ExpertMats<false>{shared, shared + (size_t)Fs * L, shared + 2 * (size_t)Fs * L};
        } else {
            c.F = F;
            c.em = ExpertMats<MX>::make(experts, rec_bytes, t.seg, F, L);
        }
        return true;
    }
    __device__ int n_rows(const Ctx& c) const { return c.F; }
    __device__ int k_steps(const Ctx&) const { return L / 32; }
    __device__ RowW row_w(const Ctx& c, int n) const {
        RowW r;
        r.sh = c.seg == seg.E;
        if (n >= c.F) {
            r.g = WRow<MX>{};
            r.u = WRow<MX>{};
            r.sg = r.su = WRow<false>{nullptr};
            r.sh = true;
        } else if (r.sh) {
            r.sg = c.sm.gate(n, L);
            r.su = c.sm.up(n, L);
        } else {
            r.g = c.em.gate(n, L);
            r.u = c.em.up(n, L);
        }
        return r;
    }
    __device__ RowX row_x(const Ctx& c, int j) const {
        return j < c.nrows ? z16 + (size_t)seg.token_of(c.seg, c.row0 + j) * L : nullptr;
    }
    __device__ uint4 load_w(const Ctx&, const RowW& r, int m, int s, int kq) const {
        if (r.sh) return m == 0 ? r.sg.load(s, kq) : r.su.load(s, kq);
        return m == 0 ? r.g.load(s, kq) : r.u.load(s, kq);
    }
    __device__ XFrag load_x(const Ctx&, RowX r, int s, int kq) const { return r ? ld16(r + s * 32 + kq * 8) : zero4(); }
    __device__ static f32x4 mma(f32x4 a, uint4 w, XFrag x) { return mfma16(w, x, a); }
    __device__ void epilogue(const Ctx& c, int n, int j, const float* v) const {
        if (n < c.F && j < c.nrows) H[(size_t)(c.row0 + j) * Hs + n] = (uint16_t)f2bf(silu(v[0]) * v[1]);
    }
};

template <bool MX>
struct StreamDown {
    SegSpace seg;
    const uint16_t* H;
    const void* experts;
    size_t rec_bytes;
    const uint16_t* shared;
    int L, F, Fs, Hs;
    float* Y;
    struct Ctx { int seg, row0, nrows, F; ExpertMats<MX> em; ExpertMats<false> sm; };
    struct RowW { WRow<MX> d; WRow<false> sd; bool sh; };
    typedef const uint16_t* RowX;
    typedef uint4 XFrag;
    __device__ bool tile(int by, Ctx& c) const {
        if (by >= *seg.ntiles) return false;
        const Tile t = seg.tiles[by];
        c.seg = t.seg;
        c.row0 = t.row0;
        c.nrows = t.nrows;
        if (t.seg == seg.E) {
            c.F = Fs;
            c.sm = ExpertMats<false>{shared, shared + (size_t)Fs * L, shared + 2 * (size_t)Fs * L};
        } else {
            c.F = F;
            c.em = ExpertMats<MX>::make(experts, rec_bytes, t.seg, F, L);
        }
        return true;
    }
    __device__ int n_rows(const Ctx&) const { return L; }
    __device__ int k_steps(const Ctx& c) const { return c.F / 32; }
    __device__ RowW row_w(const Ctx& c, int n) const {
        RowW r;
        r.sh = c.seg == seg.E;
        if (n >= L) {
            r.d = WRow<MX>{};
            r.sd = WRow<false>{nullptr};
            r.sh = true;
        } else if (r.sh) {
            r.sd = c.sm.down(n, c.F);
        } else {
            r.d = c.em.down(n, c.F);
        }
        return r;
    }
    __device__ RowX row_x(const Ctx& c, int j) const { return j < c.nrows ? H + (size_t)(c.row0 + j) * Hs : nullptr; }
    __device__ uint4 load_w(const Ctx&, const RowW& r, int, int s, int kq) const { return r.sh ? r.sd.load(s, kq) : r.d.load(s, kq); }
    __device__ XFrag load_x(const Ctx&, RowX r, int s, int kq) const { return r ? ld16(r + s * 32 + kq * 8) : zero4(); }
    __device__ static f32x4 mma(f32x4 a, uint4 w, XFrag x) { return mfma16(w, x, a); }
    __device__ void epilogue(const Ctx& c, int n, int j, const float* v) const {
        if (n >= L || j >= c.nrows) return;
        const int drow = seg.dest_of(c.seg, c.row0 + j);
        if (drow >= 0) Y[(size_t)drow * L + n] = v[0];
    }
};

}  // namespace lmoe
