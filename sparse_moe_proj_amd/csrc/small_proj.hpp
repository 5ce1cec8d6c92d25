// Dense projection of a small batch (T <= 64 tokens): out[t][n] = sum_k x[t][k] * W[n][k].
//
// The work is reading W once from HBM.  A workgroup owns 16 weight rows; its W waves split K
// into contiguous ranges and each wave requests all weight units of its range (up to SMAX MFMA
// steps at a time) before anything else, so the whole range is in flight at once.  While those
// loads travel, the workgroup stages the activations of the first 16 tokens into LDS as bf16
// (XM = 0: a bf16 [T][K] input; XM = 1: the fp32 sum, in order, of G bf16 partial inputs [G][T][K],
// rounded once; XM = 2: bf16(RMSNorm(h)) of an fp32 residual h [T][K] with unit gain, each
// token's sum of squares taken by one wave in a fixed order), so the token operand is read from
// LDS rather than once per wave from L2.  Further groups of 16 tokens
// are staged in turn and reuse the weights held in registers.  The MFMA is
// v_mfma_f32_16x16x32_bf16 with the weights as A (16 rows) and the tokens as B (columns past T
// are zero).  The waves' partial tiles meet in LDS and are summed in wave order.  A second
// product over the same input (the two halves of the folded router) can share the launch.
#pragma once

#include "problems.hpp"

namespace lmoe {

struct SmallProj {
    const uint16_t* x16;  // XM 0: [T][K] bf16; XM 1: [G][T][K] bf16 partials (summed in fp32)
    const float* xpart;   // XM 2: the residual h [T][K] fp32
    int G;
    const uint16_t* W;    // [N][K] bf16
    int T, N, K, mode;    // mode 0: out32 = v, out16 = bf16(v); 1: out16 = bf16(v); 2: out32 += v;
                          // 3: out32[kg][T][N] = v, the product over K group kg (below)
    float* out32;
    uint16_t* out16;
    // Optional second product in the same launch (Gr != null), from Gr [E][2][K] bf16 (hi, lo
    // halves of each row): logits[h][t][e] = x[t] . Gr[e][h] (+ bias[e] for h = 0), so that
    // logits[0] + logits[1] are the router logits.  Its 2 * ceil(E / 16) row blocks (the hi
    // blocks, then the lo blocks) follow the ceil(N / 16) blocks of W.
    const uint16_t* Gr;
    const float* bias;
    int E;
    float* logits;  // [2][T][E]
    uint16_t* out16h;  // mode 0, optional: fp16(v) as well (the token operand of 4-bit experts)
    float eps = 1e-6f;  // XM 2: the RMSNorm epsilon
    // K groups (mode 3, no router rows): W and the input rows are KG * K wide; block b of the
    // KG * ceil(N / 16) row blocks multiplies columns kg * K .. of both, kg = b / ceil(N / 16).
    // Workgroup w takes the blocks of K group w % KG only (the grid is a multiple of KG), so its
    // staged input columns serve all of its blocks.
    int KG = 1;
};

// Largest staged-activation LDS a small-batch projection takes (plus W KB of static LDS).
constexpr size_t kSmallProjLds = 128 * 1024;

// Token groups of 16 (the MFMA's token columns) a launch takes: T <= 16 * kSmallProjGroups.
constexpr int kSmallProjGroups = 4;

// LDS bytes of the staged activations: one token group, 16 rows of K/8 16-byte units plus one
// unit of padding per row.
__host__ __device__ inline size_t small_proj_lds(int K) { return (size_t)16 * (K / 8 + 1) * 16; }

// Row blocks (16 weight rows each: the ceil(N / 16) blocks of W, then the router's hi and lo
// blocks) are dealt to the workgroups (block b to workgroup b % grid); a workgroup with several
// blocks requests the next block's weights before it reduces the current one, and a batch of at
// most 16 tokens is staged once for all of them.
template <int W, int SMAX, int XM>
__global__ __launch_bounds__(64 * W) void small_proj_kernel(const SmallProj p) {
    extern __shared__ uint4 xs[];  // [16][K / 8 + 1]: the current token group
    __shared__ float red[W][256];
    __shared__ float rnorm[16];  // XM 2: 1 / rms of the group's tokens
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int kq = lane >> 4, j = lane & 15;
    const int K = p.K, T = p.T;
    const int ns = K / 32;
    const int nbw = (p.N + 15) / 16, nbe = (p.E + 15) / 16;
    const int KP = p.KG * K;  // row pitch of W and of the input rows
    const int nblk = nbw * p.KG + (p.Gr ? 2 * nbe : 0);
    const int s0 = wave * ns / W, s1 = (wave + 1) * ns / W;
    // a wave's whole K range fits in the registers: every token group reuses the same weights
    const bool single = s1 - s0 <= SMAX;
    const int per = K / 8, xst = per + 1;
    const int ngroups = (T + 15) / 16;
    struct Blk {
        const uint16_t* wrow;  // this lane's weight row
        int n0, half, nrow, kg;
        bool rt;               // a router block (half 0: hi rows, 1: lo rows)
    };
    auto blk_of = [&](int b) {
        Blk o;
        o.rt = b >= nbw * p.KG;
        o.kg = o.rt ? 0 : b / nbw;
        const int rb = o.rt ? b - nbw * p.KG : b - o.kg * nbw;
        o.half = o.rt && rb >= nbe ? 1 : 0;
        o.n0 = (rb - o.half * nbe) * 16;
        o.nrow = o.rt ? p.E : p.N;
        o.wrow = o.rt ? p.Gr + ((size_t)min(o.n0 + j, o.nrow - 1) * 2 + o.half) * K
                      : p.W + (size_t)min(o.n0 + j, o.nrow - 1) * KP + (size_t)o.kg * K;
        return o;
    };
    uint4 wv[SMAX];
    auto loadw = [&](const uint16_t* wrow, int b) {
#pragma unroll
        for (int i = 0; i < SMAX; ++i)
            if (b + i < s1) wv[i] = ld16(wrow + (b + i) * 32 + kq * 8);
    };
    // this workgroup's blocks: K group kg0, row blocks r0, r0 + step, ... (KG = 1: every block)
    const int kg0 = (int)blockIdx.x % p.KG, step = (int)gridDim.x / p.KG;
    const int nrb = p.KG == 1 ? nblk : nbw;
    int r = (int)blockIdx.x / p.KG;
    int b = kg0 * nbw + r;
    Blk cur = blk_of(b);
    if (s0 < s1) loadw(cur.wrow, s0);
    bool first = true;
    int staged_kg = -1;  // the K group whose input columns are staged
    while (true) {
        const int rn = r + step;
        const bool more = rn < nrb;
        const int bn = kg0 * nbw + rn;
        const Blk nxt = blk_of(more ? bn : b);
        static_for<kSmallProjGroups>([&](auto G) {
            constexpr int g = decltype(G)::value;
            if (g < ngroups) {
                const int t0 = 16 * g, tn = min(16, T - t0);
                if (g > 0 || !first) {
                    __syncthreads();  // the previous group's or block's LDS reads are done
                    if (g > 0 && !single && s0 < s1) loadw(cur.wrow, s0);
                }
                // the staged tokens of a single group stay valid for the workgroup's next blocks of
                // the same K group
                if (ngroups > 1 || first || staged_kg != cur.kg) {
                    staged_kg = cur.kg;
                    if constexpr (XM == 2) {
                        for (int t = wave; t < tn; t += W) {
                            const float4* row = reinterpret_cast<const float4*>(p.xpart + (size_t)(t0 + t) * K);
                            float ss = 0.f;
                            for (int c = lane; c < K / 4; c += 64) {
                                const float4 u = row[c];
                                ss += u.x * u.x + u.y * u.y + u.z * u.z + u.w * u.w;
                            }
#pragma unroll
                            for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
                            if (lane == 0) rnorm[t] = 1.0f / sqrtf(ss / (float)K + p.eps);
                        }
                        __syncthreads();
                    }
                    for (int e = threadIdx.x; e < tn * per; e += 64 * W) {
                        const int t = e / per, c = e - t * per;
                        uint4 v;
                        if constexpr (XM == 0) {
                            v = ld16(p.x16 + (size_t)(t0 + t) * K + c * 8);
                        } else if constexpr (XM == 2) {
                            const float* src = p.xpart + (size_t)(t0 + t) * K + c * 8;
                            const float4 u0 = *reinterpret_cast<const float4*>(src);
                            const float4 u1 = *reinterpret_cast<const float4*>(src + 4);
                            const float r = rnorm[t];
                            v = make_uint4(pack_bf2(u0.x * r, u0.y * r), pack_bf2(u0.z * r, u0.w * r),
                                           pack_bf2(u1.x * r, u1.y * r), pack_bf2(u1.z * r, u1.w * r));
                        } else {
                            float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
                            for (int q = 0; q < p.G; ++q) {
                                const uint4 u = ld16(p.x16 + ((size_t)q * T + t0 + t) * KP + (size_t)cur.kg * K + c * 8);
                                add_bf16x8(a, u);
                            }
                            v = make_uint4(pack_bf2(a[0], a[1]), pack_bf2(a[2], a[3]), pack_bf2(a[4], a[5]),
                                           pack_bf2(a[6], a[7]));
                        }
                        xs[t * xst + c] = v;
                    }
                }
                __syncthreads();
                f32x4 acc = f32x4{};
                const bool tok = j < tn;
                for (int b2 = s0; b2 < s1; b2 += SMAX) {
                    if (b2 != s0) loadw(cur.wrow, b2);
#pragma unroll
                    for (int i = 0; i < SMAX; ++i)
                        if (b2 + i < s1) {
                            const uint4 xv = tok ? xs[j * xst + (b2 + i) * 4 + kq] : zero4();
                            acc = mfma16(wv[i], xv, acc);
                        }
                }
                // the last group: the next block's weights are requested before this one is reduced
                if (g == ngroups - 1 && more && s0 < s1) loadw(nxt.wrow, s0);
                // lane (kq, j): rows n0 + 4 kq + r, token t0 + j
#pragma unroll
                for (int r = 0; r < 4; ++r) red[wave][(4 * kq + r) * 16 + j] = acc[r];
                __syncthreads();
                // thread e: token t0 + e / 16, row n0 + e % 16 (16 consecutive outputs of a token)
                for (int e = threadIdx.x; e < 256; e += 64 * W) {
                    const int t = e >> 4, r = e & 15, n = cur.n0 + r;
                    if (t >= tn || n >= cur.nrow) continue;
                    float v = 0.f;
#pragma unroll
                    for (int w = 0; w < W; ++w) v += red[w][r * 16 + t];
                    if (cur.rt) {
                        p.logits[((size_t)cur.half * T + t0 + t) * p.E + n] = cur.half == 0 && p.bias ? v + p.bias[n] : v;
                        continue;
                    }
                    const size_t o = (size_t)(t0 + t) * p.N + n;
                    if (p.mode == 0) {
                        p.out32[o] = v;
                        p.out16[o] = (uint16_t)f2bf(v);
                        if (p.out16h) p.out16h[o] = __builtin_bit_cast(uint16_t, f16_sat(v));
                    } else if (p.mode == 1) {
                        p.out16[o] = (uint16_t)f2bf(v);
                    } else if (p.mode == 3) {
                        p.out32[(size_t)cur.kg * T * p.N + o] = v;
                    } else {
                        p.out32[o] += v;
                    }
                }
            }
        });
        if (!more) break;
        first = false;
        r = rn;
        b = bn;
        cur = nxt;
    }
}

}  // namespace lmoe

namespace lmoe {

// ==============================================================================================
// Small-batch projection with the weight rows dealt evenly over the compute units.
//
// The same product as small_proj_kernel (out[t][n] = sum_k x[t][k] W[n][k], T <= 64), for a
// launch that reads every weight byte once: the R rows (W's N rows, then, with a folded router,
// the 2E rows of Gr [E][2][K] as one [2E][K] matrix) are cut into `rpw` consecutive rows per
// workgroup, one workgroup per compute unit, so each unit streams the same share (at the 145B
// shape 11 rows of 2560 for D and the router together, 10 rows of 1792 for U) instead of whole
// 16-row blocks on some units and none on others.  A workgroup takes its rows 16 at a time as
// the MFMA's A operand (rows past its range are zero); its W waves split K into contiguous step
// ranges.  Each wave loads the token operand of its own K range straight into registers (token
// j of the group in lane j, as the B operand), issued before its weight loads, so the tokens
// arrive first and no LDS staging pass sits between the loads and the MFMAs.  The XM modes are
// those of small_proj_kernel: 0 bf16 x; 1 the in-order sum of G fp32 partial inputs, rounded
// once to bf16; 2 bf16(RMSNorm(h)) of an fp32 residual h (each token's sum of squares: per lane
// over its steps in order, over the lane's four K chunks as (a + b) + (c + d), then over the waves
// in order).  The waves' partial tiles meet in LDS and are summed in wave order.
// ==============================================================================================
constexpr int kRowsMaxG = 2;  // XM 1: partial inputs held in registers per step

// MFMA steps (32 K values) a wave holds in registers, by input mode: K <= 32 * waves * steps
// (the raw token loads of all steps, the weights and the bf16 operands are in flight together).
__host__ __device__ constexpr int rows_proj_smax(int XM) { return XM == 0 ? 12 : XM == 1 ? 7 : 10; }

struct RowsProj {
    const uint16_t* x16;  // XM 0: [T][K] bf16; XM 1: [G][T][K] bf16 partials (summed in fp32)
    const float* xf;      // XM 2: the residual h [T][K] fp32
    int G;
    const uint16_t* W;    // [N][K] bf16
    int T, N, K, mode;    // mode 0: out32 = v, out16 = bf16(v) (out16h = fp16(v) if set); 1: out16 =
                          // bf16(v); 2: out32 += v
    float* out32;
    uint16_t* out16;
    uint16_t* out16h;
    const uint16_t* Gr;   // optional [E][2][K]: logits[h][t][e] = x[t] . Gr[e][h] (+ bias[e] for h = 0)
    const float* bias;
    int E;
    float* logits;        // [2][T][E]
    int rpw;              // rows per workgroup
    float eps;            // XM 2: the RMSNorm epsilon
};

template <int W, int XM>
__global__ __launch_bounds__(64 * W) void rows_proj_kernel(const RowsProj p) {
    constexpr int kRowsSmax = rows_proj_smax(XM);
    constexpr int XR = XM == 0 ? 1 : XM == 2 ? 2 : kRowsMaxG;  // 16-byte loads per step
    __shared__ float red[W][256];
    __shared__ float ssq[W][16];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int kq = lane >> 4, j = lane & 15;
    const int K = p.K, T = p.T;
    const int ns = K / 32;
    const int s0 = wave * ns / W, nst = (wave + 1) * ns / W - s0;
    const int R = p.N + (p.Gr ? 2 * p.E : 0);
    const int rbeg = (int)blockIdx.x * p.rpw, rend = min(R, rbeg + p.rpw);
    const int ngroups = (T + 15) / 16;
    uint4 xr[kRowsSmax][XR];
    uint4 wv[kRowsSmax];
    uint4 xv[kRowsSmax];

    // the token operand of group g: raw loads of token t0 + j, K chunk kq of every step
    auto load_x = [&](int g) {
        const int t = 16 * g + j;
        const bool ok = t < T;
#pragma unroll
        for (int i = 0; i < kRowsSmax; ++i) {
            if (i >= nst) break;
            const int k0 = (s0 + i) * 32 + kq * 8;
            if constexpr (XM == 0) {
                xr[i][0] = ok ? ld16(p.x16 + (size_t)t * K + k0) : zero4();
            } else if constexpr (XM == 2) {
                const float* src = p.xf + (size_t)t * K + k0;
                xr[i][0] = ok ? ld16(src) : zero4();
                xr[i][1] = ok ? ld16(src + 4) : zero4();
            } else {
#pragma unroll
                for (int q = 0; q < kRowsMaxG; ++q)
                    xr[i][q] = ok && q < p.G ? ld16(p.x16 + ((size_t)q * T + t) * K + k0) : zero4();
            }
        }
    };
    // raw loads -> bf16 B operands (XM 2: needs every wave's sum of squares; one barrier)
    auto make_x = [&]() {
        if constexpr (XM == 0) {
#pragma unroll
            for (int i = 0; i < kRowsSmax; ++i)
                if (i < nst) xv[i] = xr[i][0];
        } else if constexpr (XM == 1) {
#pragma unroll
            for (int i = 0; i < kRowsSmax; ++i) {
                if (i >= nst) break;
                float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int q = 0; q < kRowsMaxG; ++q) add_bf16x8(a, xr[i][q]);
                xv[i] = make_uint4(pack_bf2(a[0], a[1]), pack_bf2(a[2], a[3]), pack_bf2(a[4], a[5]), pack_bf2(a[6], a[7]));
            }
        } else {
            float ss = 0.f;
#pragma unroll
            for (int i = 0; i < kRowsSmax; ++i) {
                if (i >= nst) break;
                const float* u = reinterpret_cast<const float*>(&xr[i][0]);
                const float* v = reinterpret_cast<const float*>(&xr[i][1]);
#pragma unroll
                for (int c = 0; c < 4; ++c) ss += u[c] * u[c];
#pragma unroll
                for (int c = 0; c < 4; ++c) ss += v[c] * v[c];
            }
            // lanes j, j + 16, j + 32, j + 48 hold token j's K chunks 0..3: lane j sums them in order
            const float b = __shfl_xor(ss, 16), c = __shfl_xor(ss, 32), d = __shfl_xor(ss, 48);
            if (kq == 0) ssq[wave][j] = (ss + b) + (c + d);
            __syncthreads();
            float tot = 0.f;
#pragma unroll
            for (int w = 0; w < W; ++w) tot += ssq[w][j];
            const float r = 1.0f / sqrtf(tot / (float)K + p.eps);
#pragma unroll
            for (int i = 0; i < kRowsSmax; ++i) {
                if (i >= nst) break;
                const float* u = reinterpret_cast<const float*>(&xr[i][0]);
                const float* v2 = reinterpret_cast<const float*>(&xr[i][1]);
                xv[i] = make_uint4(pack_bf2(u[0] * r, u[1] * r), pack_bf2(u[2] * r, u[3] * r), pack_bf2(v2[0] * r, v2[1] * r),
                                   pack_bf2(v2[2] * r, v2[3] * r));
            }
        }
    };
    auto wrow = [&](int n) -> const uint16_t* {
        return n < p.N ? p.W + (size_t)n * K : p.Gr + (size_t)(n - p.N) * K;
    };
    auto load_w = [&](int n0) {
        const int nr = min(16, rend - n0);
        const bool rv = j < nr;
        const uint16_t* wr = wrow(n0 + (rv ? j : 0));
#pragma unroll
        for (int i = 0; i < kRowsSmax; ++i) {
            if (i >= nst) break;
            wv[i] = rv ? ld16(wr + (s0 + i) * 32 + kq * 8) : zero4();
        }
    };

    if (rbeg >= rend) return;
    load_x(0);  // tokens first: they are needed by every MFMA
    load_w(rbeg);
    bool have_x = false;  // xv holds group 0 (kept across blocks when there is one group)
    for (int n0 = rbeg; n0 < rend; n0 += 16) {
        const int nr = min(16, rend - n0);
        for (int g = 0; g < ngroups; ++g) {
            const int t0 = 16 * g, tn = min(16, T - t0);
            if (!(have_x && ngroups == 1)) {
                if (n0 != rbeg || g != 0) load_x(g);
                make_x();
                have_x = true;
            }
            f32x4 acc = f32x4{};
#pragma unroll
            for (int i = 0; i < kRowsSmax; ++i)
                if (i < nst) acc = mfma16(wv[i], xv[i], acc);
            // the next block's weights are requested before this one is reduced
            if (g == ngroups - 1 && n0 + 16 < rend) load_w(n0 + 16);
#pragma unroll
            for (int r = 0; r < 4; ++r) red[wave][(4 * kq + r) * 16 + j] = acc[r];
            __syncthreads();
            if (threadIdx.x < 256) {
                const int t = threadIdx.x >> 4, r = threadIdx.x & 15, n = n0 + r;
                if (t < tn && r < nr) {
                    float v = 0.f;
#pragma unroll
                    for (int w = 0; w < W; ++w) v += red[w][r * 16 + t];
                    if (n >= p.N) {
                        const int q = n - p.N, e = q >> 1, h = q & 1;
                        p.logits[((size_t)h * T + t0 + t) * p.E + e] = h == 0 && p.bias ? v + p.bias[e] : v;
                    } else {
                        const size_t o = (size_t)(t0 + t) * p.N + n;
                        if (p.mode == 0) {
                            p.out32[o] = v;
                            p.out16[o] = (uint16_t)f2bf(v);
                            if (p.out16h) p.out16h[o] = __builtin_bit_cast(uint16_t, f16_sat(v));
                        } else if (p.mode == 1) {
                            p.out16[o] = (uint16_t)f2bf(v);
                        } else {
                            p.out32[o] += v;
                        }
                    }
                }
            }
            __syncthreads();  // red (and ssq) are reused
        }
    }
}

}  // namespace lmoe
