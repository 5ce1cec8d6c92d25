// Expert GEMMs of large MXFP4 batches on the CDNA4 block-scaled MFMA (v_mfma_scale_f32_32x32x64_f8f6f4).
//
// The routed experts' gate/up and down products take their MXFP4 records as they are stored
// (E2M1 values with one E8M0 scale per 32 values along K) as the B operand, and the activations
// as MXFP8 (E4M3 values with one E8M0 scale per 32 values of a row) plus the MXFP4 residual of
// that rounding as two A operands: z is quantized once per token, H (written in bf16 by the
// gate/up epilogue) once per routed row.  The MFMA applies both block scales, so no 4-bit value
// is decoded in software.
//
// Operand lane layouts of the 32x32x64 form with A in FP8 and B in FP4 (lane l, g = l / 32):
//   A: row l % 32; bytes 0..15 hold K 16g .. 16g + 15, bytes 16..31 hold K 32 + 16g .. 32 + 16g + 15;
//   B: row l % 32; 16 bytes hold K 32g .. 32g + 31 (low nibble first);
//   scales: lane l gives the E8M0 scale of row l % 32 for the 32-value block g of K, in the byte
//   of its scale register that the instruction's op_sel picks;
//   D: as for the bf16 32x32 MFMAs (register r of lane l: row 8 (r / 4) + 4 g + r % 4, column l % 32).
//
// The pipelined structure follows the bf16 kernel (gemm_pipe.hpp): one workgroup of WR x WC waves
// per BM x BN tile, stages of 128 K values copied straight into LDS by global_load_lds, NS stages
// deep, one barrier per stage, persistent workgroups.  A stage holds
//   A: BM rows x 128 bytes (row-major, 16-byte chunks swizzled by (row >> 1) & 7);
//   B: BN / 16 packed 1 KB tiles (16 rows x 128 values: unit (row j, 32-value block q) at 16 q + j);
//   the A scales (4 bytes per row, dword copies by BM / 64 waves) and the B scale tiles (64 bytes
//   per 16-row block, one byte per unit in the same order; one 16-byte-per-lane copy by one wave);
//   the waits of the waves that copy no scales count one copy fewer per stage;
//   with LO, a second A operand: the residual of each activation row after its MXFP8 rounding,
//   as MXFP4 (BM rows x 64 bytes, copied into packed-tile order like B) and its scales, so that
//   z = hi + lo (and H = hi + lo) carries about 6 significant bits instead of 4 (see quant_mx_kernel).
#pragma once

#include "gemm_pipe.hpp"
#include "problems.hpp"

namespace lmoe {

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

template <int BM, int BN, int NS, int WR, int WC, bool LO>
struct MxShape {
    static constexpr bool kLo = LO;
    static constexpr int kBM = BM, kBN = BN, kNS = NS;
    static constexpr int kWR = WR, kWC = WC, kWaves = WR * WC, kThreads = 64 * WR * WC;
    static constexpr int kWM = BM / WR, kWN = BN / WC;
    static constexpr int kMB = kWM / 32, kNB = kWN / 32;
    static constexpr int kAI = BM / 8, kBI = BN / 16;  // 1 KB copies per stage
    static constexpr int kAIW = kAI / kWaves, kBIW = kBI / kWaves;
    static_assert(kAI % kWaves == 0 && kBI % kWaves == 0, "copies split over the waves");
    static constexpr int kSAW = BM / 64;  // waves copying A scales (then one wave the B scales)
    static_assert(BN == 256, "the B scale tiles of a stage are one 1 KB copy");
    static_assert(kSAW + 1 + (LO ? kSAW : 0) <= kWaves, "one scale copy per wave");
    static constexpr int kLI = LO ? BM / 16 : 0, kLIW = kLI / kWaves;  // residual copies (1 KB: 16 rows)
    static_assert(!LO || kLI % kWaves == 0, "residual copies split over the waves");
    static constexpr int kSW = kSAW + 1 + (LO ? kSAW : 0);  // waves that copy scales
    static constexpr int kLoadsPerStage = kAIW + kBIW + 1 + kLIW;  // of such a wave (the others: one fewer)
    // 16-byte units of a stage: A, B, one 256-byte scale block per wave, the residual operand
    static constexpr int kAU = BM * 8, kBU = BN * 4, kSU = kWaves * 16, kLU = LO ? BM * 4 : 0;
    static constexpr int kStageUnits = kAU + kBU + kSU + kLU;
    static_assert(NS * kStageUnits * 16 <= 160 * 1024, "LDS budget");
    static_assert(kMB == 2 && kNB == 2, "64 x 64 wave tiles");
};

// Bytes one stage advances: an A row 128 values, a B tile 1 KB, A scales 4, a B scale tile 64, a
// residual row 64.
constexpr int kMxAStep = 128, kMxBStep = 1024, kMxSAStep = 4, kMxSBStep = 64, kMxLStep = 64;

__device__ __forceinline__ void lds_copy4(const void* g, uint4* lds_block) {
    __builtin_amdgcn_global_load_lds(g, (lds_ptr_t)lds_block, 4, 0, 0);
}

template <class S>
struct MxCopies {
    const uint8_t* abase;
    const uint8_t* bbase;
    const uint8_t* sbase;  // this wave's scale source
    const uint8_t* lbase;  // residual operand (LO)
    uint32_t as[S::kAIW], bs[S::kBIW], ls[S::kLIW > 0 ? S::kLIW : 1], ss;
    int sstep, sdst;  // scale source step per stage; destination (16-byte units past A and B)
};

// Copy sources: P gives a_base/b_base, src_a/src_b as for the bf16 kernel (A rows of 128 bytes,
// B 1 KB tiles), and scale_src(ctx, wave, lane, base, off, step) for the wave's scale copy.
template <class S, class P>
__device__ __forceinline__ MxCopies<S> mx_copies(const P& p, const typename P::Ctx& ctx, int wave, int lane) {
    MxCopies<S> c;
    c.abase = p.a_base(ctx);
    c.bbase = p.b_base(ctx);
#pragma unroll
    for (int i = 0; i < S::kAIW; ++i) c.as[i] = p.src_a(ctx, wave * S::kAIW + i, lane);
#pragma unroll
    for (int i = 0; i < S::kBIW; ++i) c.bs[i] = p.src_b(ctx, wave * S::kBIW + i, lane);
    p.scale_src(ctx, wave, lane, c.sbase, c.ss, c.sstep);
    // A scales (rows 64 w ..), the B scale tiles, then the residual's scales (rows 64 (w - kSAW - 1) ..)
    c.sdst = wave <= S::kSAW ? wave * 16 : S::kSAW * 16 + S::kBN / 4 + (wave - S::kSAW - 1) * 16;
    if constexpr (S::kLo) {
        c.lbase = p.lo_base(ctx);
#pragma unroll
        for (int i = 0; i < S::kLIW; ++i) c.ls[i] = p.src_lo(ctx, wave * S::kLIW + i, lane);
    }
    return c;
}

template <class S>
__device__ __forceinline__ void mx_issue(const MxCopies<S>& c, uint4* buf, int kt, int wave) {
#pragma unroll
    for (int i = 0; i < S::kAIW; ++i)
        lds_copy16(c.abase + (c.as[i] + (uint32_t)(kt * kMxAStep)), buf + (wave * S::kAIW + i) * 64);
#pragma unroll
    for (int i = 0; i < S::kBIW; ++i)
        lds_copy16(c.bbase + (c.bs[i] + (uint32_t)(kt * kMxBStep)), buf + S::kAU + (wave * S::kBIW + i) * 64);
    if (wave < S::kSW) {
        const uint8_t* g = c.sbase + (c.ss + (uint32_t)(kt * c.sstep));
        if (wave == S::kSAW)
            lds_copy16(g, buf + S::kAU + S::kBU + c.sdst);
        else
            lds_copy4(g, buf + S::kAU + S::kBU + c.sdst);
    }
    if constexpr (S::kLo) {
#pragma unroll
        for (int i = 0; i < S::kLIW; ++i)
            lds_copy16(c.lbase + (c.ls[i] + (uint32_t)(kt * kMxLStep)),
                       buf + S::kAU + S::kBU + S::kSU + (wave * S::kLIW + i) * 64);
    }
}

template <class S>
__device__ __forceinline__ void mx_prologue(const MxCopies<S>& c, int nk, uint4* st0, uint4* st1, uint4* st2,
                                            int wave) {
    if (nk > 0) mx_issue<S>(c, st0, 0, wave);
    if constexpr (S::kNS >= 3)
        if (nk > 1) mx_issue<S>(c, st1, 1, wave);
    if constexpr (S::kNS == 4)
        if (nk > 2) mx_issue<S>(c, st2, 2, wave);
}

// The scale reads of one stage (2 A rows: one dword each; 2 B rows: the bytes of blocks g and
// 2 + g), in one asm block that also waits for them (early-clobber outputs): the copies into the
// other stage buffers are in flight meanwhile, and the block keeps the compiler from waiting for
// them as well.
__device__ __forceinline__ void mx_read_scales(uint32_t a0, uint32_t a1, uint32_t b00, uint32_t b01, uint32_t b10,
                                               uint32_t b11, uint32_t (&sa)[2], uint32_t (&sb)[2][2]) {
    __asm__ volatile(
        "ds_read_b32 %0, %6\n\t"
        "ds_read_b32 %1, %7\n\t"
        "ds_read_u8 %2, %8\n\t"
        "ds_read_u8 %3, %9\n\t"
        "ds_read_u8 %4, %10\n\t"
        "ds_read_u8 %5, %11\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(sa[0]), "=&v"(sa[1]), "=&v"(sb[0][0]), "=&v"(sb[0][1]), "=&v"(sb[1][0]), "=&v"(sb[1][1])
        : "v"(a0), "v"(a1), "v"(b00), "v"(b01), "v"(b10), "v"(b11));
}

// The operand reads of one 64-K step: two 16-byte halves per A fragment, one unit per B fragment.
__device__ __forceinline__ void mx_read_frags(const uint32_t (&aa)[2][2], const uint32_t (&ba)[2], uint4 (&af)[2][2],
                                              uint4 (&bf)[2]) {
    __asm__ volatile(
        "ds_read_b128 %0, %6\n\t"
        "ds_read_b128 %1, %7\n\t"
        "ds_read_b128 %2, %8\n\t"
        "ds_read_b128 %3, %9\n\t"
        "ds_read_b128 %4, %10\n\t"
        "ds_read_b128 %5, %11\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(af[0][0]), "=&v"(af[0][1]), "=&v"(af[1][0]), "=&v"(af[1][1]), "=&v"(bf[0]), "=&v"(bf[1])
        : "v"(aa[0][0]), "v"(aa[0][1]), "v"(aa[1][0]), "v"(aa[1][1]), "v"(ba[0]), "v"(ba[1]));
}

// With the residual operand: its two units and its two scale dwords join the reads.
__device__ __forceinline__ void mx_read_scales_lo(uint32_t l0, uint32_t l1, uint32_t (&sl)[2]) {
    __asm__ volatile(
        "ds_read_b32 %0, %2\n\t"
        "ds_read_b32 %1, %3\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(sl[0]), "=&v"(sl[1])
        : "v"(l0), "v"(l1));
}
__device__ __forceinline__ void mx_read_frags_lo(const uint32_t (&aa)[2][2], const uint32_t (&ba)[2],
                                                 const uint32_t (&la)[2], uint4 (&af)[2][2], uint4 (&bf)[2],
                                                 uint4 (&lf)[2]) {
    __asm__ volatile(
        "ds_read_b128 %0, %8\n\t"
        "ds_read_b128 %1, %9\n\t"
        "ds_read_b128 %2, %10\n\t"
        "ds_read_b128 %3, %11\n\t"
        "ds_read_b128 %4, %12\n\t"
        "ds_read_b128 %5, %13\n\t"
        "ds_read_b128 %6, %14\n\t"
        "ds_read_b128 %7, %15\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(af[0][0]), "=&v"(af[0][1]), "=&v"(af[1][0]), "=&v"(af[1][1]), "=&v"(bf[0]), "=&v"(bf[1]),
          "=&v"(lf[0]), "=&v"(lf[1])
        : "v"(aa[0][0]), "v"(aa[0][1]), "v"(aa[1][0]), "v"(aa[1][1]), "v"(ba[0]), "v"(ba[1]), "v"(la[0]),
          "v"(la[1]));
}

// FP4 A x FP4 B (the residual term), both block-scaled.
template <int OPA>
__device__ __forceinline__ f32x16 mfma_mx44(const uint4& a, const uint4& b, uint32_t sa, uint32_t sb, f32x16 c) {
    const i32x8 a8 = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
    const i32x8 b8 = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c, 4, 4, OPA, (int)sa, 0, (int)sb);
}

// FP8 A x FP4 B, both block-scaled; OPA picks the byte of sa that holds this lane's A scale.
template <int OPA>
__device__ __forceinline__ f32x16 mfma_mx(const uint4& alo, const uint4& ahi, const uint4& b, uint32_t sa,
                                          uint32_t sb, f32x16 c) {
    const i32x8 a8 = {(int)alo.x, (int)alo.y, (int)alo.z, (int)alo.w, (int)ahi.x, (int)ahi.y, (int)ahi.z, (int)ahi.w};
    const i32x8 b8 = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c, 0, 4, OPA, (int)sa, 0, (int)sb);
}

template <class S>
__device__ __forceinline__ void mx_k_loop(const MxCopies<S>& c, int nk, f32x16 (&acc)[2][2], uint4* st0, uint4* st1,
                                          uint4* st2, uint4* st3, int wave, int lane) {
    constexpr int NS = S::kNS;
    constexpr int LPS = S::kLoadsPerStage;
    static_assert(NS >= 2 && NS <= 4, "two to four stages");
    const int wm = wave / S::kWC, wn = wave % S::kWC;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
    const int fr = lane & 31, g = lane >> 5;
    int arow[2], brow[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) arow[i] = wm * S::kWM + i * 32 + fr;
#pragma unroll
    for (int j = 0; j < 2; ++j) brow[j] = wn * S::kWN + j * 32 + fr;

    auto compute = [&](const uint4* buf) {
        const uint32_t A = lds_addr(buf);
        const uint32_t B = A + S::kAU * 16;
        const uint32_t SA = B + S::kBU * 16;
        const uint32_t SB = SA + S::kBM * 4;
        uint32_t sa[2], sb[2][2];
        mx_read_scales(SA + arow[0] * 4, SA + arow[1] * 4, SB + (brow[0] >> 4) * 64 + g * 16 + (brow[0] & 15),
                       SB + (brow[0] >> 4) * 64 + (2 + g) * 16 + (brow[0] & 15),
                       SB + (brow[1] >> 4) * 64 + g * 16 + (brow[1] & 15),
                       SB + (brow[1] >> 4) * 64 + (2 + g) * 16 + (brow[1] & 15), sa, sb);
        // byte 2s of the shifted A dword is block 2s + g of the row
        sa[0] >>= 8 * g;
        sa[1] >>= 8 * g;
        const uint32_t AL = SB + S::kBN * 4;  // residual scales (the waves after the B scales)
        const uint32_t AO = A + (S::kAU + S::kBU + S::kSU) * 16;
        uint32_t sl[2] = {0, 0};
        if constexpr (S::kLo) {
            mx_read_scales_lo(AL + arow[0] * 4, AL + arow[1] * 4, sl);
            sl[0] >>= 8 * g;
            sl[1] >>= 8 * g;
        }
        static_for<2>([&](auto sc) {
            constexpr int s = decltype(sc)::value;
            uint32_t aa[2][2], ba[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int sw = (arow[i] >> 1) & 7;
                aa[i][0] = A + 16 * (arow[i] * 8 + ((4 * s + g) ^ sw));
                aa[i][1] = A + 16 * (arow[i] * 8 + ((4 * s + 2 + g) ^ sw));
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) ba[j] = B + 16 * ((brow[j] >> 4) * 64 + (2 * s + g) * 16 + (brow[j] & 15));
            uint4 af[2][2], bfv[2];
            if constexpr (S::kLo) {
                uint32_t la[2];
#pragma unroll
                for (int i = 0; i < 2; ++i) la[i] = AO + 16 * ((arow[i] >> 4) * 64 + (2 * s + g) * 16 + (arow[i] & 15));
                uint4 lf[2];
                mx_read_frags_lo(aa, ba, la, af, bfv, lf);
                // the four products of z's MXFP8 part, then the four of its residual, so that no
                // MFMA waits for the one before it
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        acc[i][j] = mfma_mx<2 * s>(af[i][0], af[i][1], bfv[j], sa[i], sb[j][s], acc[i][j]);
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        acc[i][j] = mfma_mx44<2 * s>(lf[i], bfv[j], sl[i], sb[j][s], acc[i][j]);
            } else {
                mx_read_frags(aa, ba, af, bfv);
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        acc[i][j] = mfma_mx<2 * s>(af[i][0], af[i][1], bfv[j], sa[i], sb[j][s], acc[i][j]);
            }
        });
    };

    const bool scale_wave = wave < S::kSW;
#define LMOE_MX_STEP(S_, CUR_, NEXT_)                                            \
    if (kt + S_ < nk) {                                                          \
        if (scale_wave)                                                          \
            wait_stage<LPS, NS>(min(nk - 1 - (kt + S_), NS - 2));                \
        else                                                                     \
            wait_stage<LPS - 1, NS>(min(nk - 1 - (kt + S_), NS - 2));            \
        stage_barrier();                                                         \
        if (kt + S_ + NS - 1 < nk) mx_issue<S>(c, NEXT_, kt + S_ + NS - 1, wave); \
        compute(CUR_);                                                           \
    }
    if constexpr (NS == 4) {
        for (int kt = 0; kt < nk; kt += 4) {
            LMOE_MX_STEP(0, st0, st3)
            LMOE_MX_STEP(1, st1, st0)
            LMOE_MX_STEP(2, st2, st1)
            LMOE_MX_STEP(3, st3, st2)
        }
    } else if constexpr (NS == 3) {
        for (int kt = 0; kt < nk; kt += 3) {
            LMOE_MX_STEP(0, st0, st2)
            LMOE_MX_STEP(1, st1, st0)
            LMOE_MX_STEP(2, st2, st1)
        }
    } else {
        for (int kt = 0; kt < nk; kt += 2) {
            LMOE_MX_STEP(0, st0, st1)
            LMOE_MX_STEP(1, st1, st0)
        }
    }
#undef LMOE_MX_STEP
}

// Persistent workgroups over the (M tile, N tile) pairs, XCD-grouped and overlapped with the
// next tile's first stages as in pipe_gemm_persistent.
template <class S, class P>
__global__ __launch_bounds__(S::kThreads) void mx_gemm_persistent(const P p, int n_tiles) {
    __shared__ uint4 st0[S::kStageUnits], st1[S::kStageUnits];
    __shared__ uint4 st2[S::kNS >= 3 ? S::kStageUnits : 1], st3[S::kNS == 4 ? S::kStageUnits : 1];
    const int total = p.m_tiles() * n_tiles;
    const int gx = min(8, (int)gridDim.x);
    const int x = blockIdx.x % gx, wi = blockIdx.x / gx;
    const int nwx = ((int)gridDim.x - x + gx - 1) / gx;
    const int lo = (int)((long)total * x / gx), hi = (int)((long)total * (x + 1) / gx);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rb = (wave / S::kWC) * S::kWM, cb = (wave % S::kWC) * S::kWN;

    auto next_tile = [&](int& l, typename P::Ctx& ctx) {
        for (; l < hi; l += nwx)
            if (p.tile(l / n_tiles, l % n_tiles, ctx)) return true;
        return false;
    };
    int l = lo + wi;
    typename P::Ctx ctx;
    if (!next_tile(l, ctx)) return;
    int nk = p.k_stages(ctx);
    MxCopies<S> c = mx_copies<S>(p, ctx, wave, lane);
    mx_prologue<S>(c, nk, st0, st1, st2, wave);
    f32x16 acc[2][2];
    while (true) {
        mx_k_loop<S>(c, nk, acc, st0, st1, st2, st3, wave, lane);
        const auto prep = p.template prep<2>(ctx, rb, lane);
        int ln = l + nwx;
        typename P::Ctx nctx;
        const bool more = next_tile(ln, nctx);
        int nnk = 0;
        MxCopies<S> nc;
        if (more) {
            nnk = p.k_stages(nctx);
            nc = mx_copies<S>(p, nctx, wave, lane);
        }
        stage_barrier();
        if (more) mx_prologue<S>(nc, nnk, st0, st1, st2, wave);
        p.template store<2, 2>(ctx, acc, prep, rb, cb, lane);
        if (!more) break;
        l = ln;
        ctx = nctx;
        nk = nnk;
        c = nc;
    }
}

// ---------------------------------------------------------------------------------------------
// MXFP8 encoding (OCP Microscaling Formats v1.0 block layout: 32 E4M3 values sharing one E8M0
// scale).  The scale is the smallest power of two 2^E with amax / 2^E <= 448 (E4M3's largest
// value), so no value of the block saturates: E = floor(log2(amax)) - 8, plus one when amax's
// significand exceeds 1.75.  (The specification's own choice, floor(log2(amax)) - 8 alone, maps
// the largest value into [256, 512) and clamps it to 448 in about a fifth of the blocks.)  Each
// value divided by the scale is rounded to the nearest E4M3 value, ties to even.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t mx8_scale_bits(float amax) {
    const uint32_t u = __float_as_uint(amax);
    const int eb = (int)((u >> 23) & 0xFF);  // biased exponent of amax
    return (uint32_t)max(eb - 8 + ((u & 0x7FFFFFu) > 0x600000u ? 1 : 0), 0);
}
// 1 / scale for a biased scale exponent sb (0 .. 246)
__device__ __forceinline__ float mx8_inv_scale(uint32_t sb) { return __uint_as_float((254u - sb) << 23); }

// MXFP4 scale: the smallest power of two 2^E with amax / 2^E <= 6 (as mx8_scale_bits, for E2M1)
__device__ __forceinline__ uint32_t mx4_scale_bits(float amax) {
    const uint32_t u = __float_as_uint(amax);
    const int eb = (int)((u >> 23) & 0xFF);
    return (uint32_t)max(eb - 2 + ((u & 0x7FFFFFu) > 0x400000u ? 1 : 0), 0);
}

// z (bf16 [rows][K], K % 32 == 0, rows contiguous) -> MXFP8: E4M3 [rows][K] and E8M0 [rows][K / 32];
// with q4 (two-term form), also the residual z - MXFP8(z) (exact in fp32) as MXFP4: E2M1
// [rows][K / 2] (low nibble = even K) and E8M0 [rows][K / 32].  One thread per block of 32 values;
// a workgroup's 256 blocks (16 KB) are read with coalesced loads into LDS first, chunk c of block t
// at 4 t + ((c + t / 4) & 3): the 16 lanes of one 16-byte read then hit 16 different 16-byte bank
// groups, so the per-thread reads are free of bank conflicts.
__global__ __launch_bounds__(256) void quant_mx_kernel(const uint16_t* __restrict__ src, size_t nblocks,
                                                       uint8_t* __restrict__ q, uint8_t* __restrict__ qs,
                                                       uint8_t* __restrict__ q4, uint8_t* __restrict__ q4s) {
    __shared__ uint4 sm[1024];
    const size_t b0 = (size_t)blockIdx.x * 256;
    const int nb = (int)min((size_t)256, nblocks - b0);
    const uint4* in = reinterpret_cast<const uint4*>(src + b0 * 32);
    for (int j = threadIdx.x; j < nb * 4; j += 256) sm[(j & ~3) | (((j & 3) + (j >> 4)) & 3)] = in[j];
    __syncthreads();
    const int t = threadIdx.x;
    if (t >= nb) return;
    const size_t b = b0 + t;
    uint4 w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = sm[4 * t + ((i + (t >> 2)) & 3)];
    float v[32];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t u[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[8 * i + 2 * j] = bf2f(u[j] & 0xFFFFu);
            v[8 * i + 2 * j + 1] = bf2f(u[j] >> 16);
        }
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    const uint32_t sb = mx8_scale_bits(amax);
    const float inv = mx8_inv_scale(sb);
    // E4M3 codes by the conversion instruction, four per dword (first value in the low byte); it
    // rounds to nearest even as the software rounding of the format does (checked bit for bit on
    // every bf16 value of the range and the fp32 values beside each), and |v / scale| <= 448 by
    // the choice of the scale, so nothing saturates
    uint32_t c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * i] * inv, v[4 * i + 1] * inv, 0, false);
        c[i] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v[4 * i + 2] * inv, v[4 * i + 3] * inv, lo, true);
    }
    uint4* out = reinterpret_cast<uint4*>(q + b * 32);
    out[0] = make_uint4(c[0], c[1], c[2], c[3]);
    out[1] = make_uint4(c[4], c[5], c[6], c[7]);
    qs[b] = (uint8_t)sb;
    if (!q4) return;
    const float scale = e8m0_to_f32(sb);
    float r[32], ramax = 0.f;
    static_for<32>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        r[i] = v[i] - __builtin_amdgcn_cvt_f32_fp8((int)c[i / 4], i % 4) * scale;
        ramax = fmaxf(ramax, fabsf(r[i]));
    });
    const uint32_t s4 = mx4_scale_bits(ramax);
    const float inv4 = mx8_inv_scale(s4);
    // E2M1 codes two per byte (even value in the low nibble), by the conversion instruction with a
    // unit scale on the pre-scaled values (|r / scale| <= 6 by the choice of the scale)
    int n[4] = {0, 0, 0, 0};
    static_for<16>([&](auto mc) {
        constexpr int m = decltype(mc)::value;
        n[m / 4] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(n[m / 4], r[2 * m] * inv4, r[2 * m + 1] * inv4, 1.0f, m % 4);
    });
    *reinterpret_cast<uint4*>(q4 + b * 16) = make_uint4((uint32_t)n[0], (uint32_t)n[1], (uint32_t)n[2], (uint32_t)n[3]);
    q4s[b] = (uint8_t)s4;
}

// ---------------------------------------------------------------------------------------------
// Problems.  Both take the routed tiles of the work list only (seg.part = 1); the shared expert's
// bf16 segment runs in the bf16 kernels.  MXFP4 record of F x L gate/up and L x F down (see
// ExpertRows): nibbles gate, up, down (F L / 2 bytes each), then scales gate, up, down
// (F L / 32 bytes each); packed nibble tile (16-row block nb, 128-value group kg) at
// nb * 8 K + kg * 1024 of its matrix, its scale tile at nb * K / 2 + kg * 64 of its scale matrix.
// ---------------------------------------------------------------------------------------------

// Gate/up: H = bf16(SiLU(z gate^T) * (z up^T)) over routed rows, z taken as its MXFP8 part plus
// its MXFP4 residual (shape with LO); the B tile of a wave column holds 32 gate rows, then the 32
// up rows of the same f.
template <class S>
struct MxUp {
    static constexpr int kHalf = S::kWN / 2;
    static constexpr int kFPerTile = S::kBN / 2;
    SegSpace seg;
    const uint8_t* z8;   // [T][zp] E4M3
    const uint8_t* z8s;  // [T][zp / 32] E8M0
    const uint8_t* z4;   // [T][zp / 2] E2M1 residual
    const uint8_t* z4s;  // [T][zp / 32] E8M0
    const uint8_t* experts;
    size_t rec;  // bytes per record
    int L, F;
    uint16_t* h16;  // [T k][F] bf16 by segment row
    struct Ctx { int seg, row0, nrows, f0; const uint8_t* r; };
    __device__ int m_tiles() const { return seg.count(); }
    __device__ bool tile(int bx, int by, Ctx& c) const {
        if (bx >= seg.count()) return false;
        const Tile t = seg.at(bx);
        c.seg = t.seg;
        c.row0 = t.row0;
        c.nrows = t.nrows;
        c.r = experts + (size_t)t.seg * rec;
        c.f0 = by * kFPerTile;
        return c.f0 < F;
    }
    __device__ int k_stages(const Ctx&) const { return L / 128; }
    __device__ const uint8_t* a_base(const Ctx&) const { return z8; }
    __device__ const uint8_t* b_base(const Ctx& c) const { return c.r; }
    __device__ uint32_t tok_off(const Ctx& c, int r) const {
        const int rr = min(r, c.nrows - 1);
        return (uint32_t)seg.z_off(c.seg, seg.token_of(c.seg, c.row0 + rr), L);
    }
    __device__ uint32_t src_a(const Ctx& c, int i, int lane) const {
        return rowmajor_off(tok_off(c, rowmajor_row(i, lane)), i, lane);
    }
    // residual: copy i takes rows 16 i .. 16 i + 15, lane (q, j) the 32 values of block q of row
    // 16 i + j, so the stage lands in packed-tile order
    __device__ const uint8_t* lo_base(const Ctx&) const { return z4; }
    __device__ uint32_t src_lo(const Ctx& c, int i, int lane) const {
        return tok_off(c, 16 * i + (lane & 15)) / 2 + (lane >> 4) * 16;
    }
    // matrix (0 gate, 1 up) and 16-row block of B-tile rows 16 b .. 16 b + 15
    __device__ void b_block(const Ctx& c, int b, int& mat, int& nb) const {
        const int r = b * 16, wc = r / S::kWN, rr = r % S::kWN;
        mat = rr >= kHalf;
        nb = min(c.f0 + wc * kHalf + rr % kHalf, F - 16) >> 4;
    }
    __device__ uint32_t src_b(const Ctx& c, int i, int lane) const {
        int mat, nb;
        b_block(c, i, mat, nb);
        return (uint32_t)((size_t)mat * F * L / 2 + (size_t)nb * 8 * L) + lane * 16;
    }
    __device__ void scale_src(const Ctx& c, int wave, int lane, const uint8_t*& base, uint32_t& off, int& step) const {
        if (wave == S::kSAW) {  // lane l: 16 bytes (units of block l % 4) of B-tile block l / 4's scales
            int mat, nb;
            b_block(c, lane >> 2, mat, nb);
            base = c.r;
            off = (uint32_t)((size_t)3 * F * L / 2 + (size_t)mat * F * L / 32 + (size_t)nb * (L / 2)) + (lane & 3) * 16;
            step = kMxSBStep;
        } else if (wave > S::kSAW) {  // residual scales of rows 64 w + lane
            const int w = wave - S::kSAW - 1;
            base = z4s;
            off = tok_off(c, w * 64 + lane) / 32;
            step = kMxSAStep;
        } else {  // A scales of rows 64 w + lane
            base = z8s;
            off = tok_off(c, wave * 64 + lane) / 32;
            step = kMxSAStep;
        }
    }
    struct Prep {};
    template <int MB>
    __device__ Prep prep(const Ctx&, int, int) const { return {}; }
    // SwiGLU in bf16 rows (quant_mx_kernel then makes H's MXFP8 part and residual for the down
    // product: one pass over H, cheaper than the block maxima and byte stores in this epilogue)
    template <int MB, int NB>
    __device__ __forceinline__ void store(const Ctx& c, f32x16 (&acc)[MB][NB], Prep, int rb, int cb, int lane) const {
        const int f = c.f0 + (cb / S::kWN) * kHalf + frag32_col(lane);
        static_for<MB>([&](auto i) {
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = rb + i * 32 + frag32_row(r, lane);
                if (m < c.nrows && f < F)
                    h16[(size_t)(c.row0 + m) * F + f] = (uint16_t)f2bf(silu(acc[i][0][r]) * acc[i][1][r]);
            }
        });
    }
};

// Down: Y[dest(p)][n] = bf16(H[p] . down[n]) over routed rows, H taken as its MXFP8 part plus
// (shape with LO) its MXFP4 residual.
template <class S>
struct MxDown {
    SegSpace seg;
    const uint8_t* h8;
    const uint8_t* h8s;
    const uint8_t* h4;   // residual (LO)
    const uint8_t* h4s;
    const uint8_t* experts;
    size_t rec;
    int L, F;
    uint16_t* Y;  // [T k + T][L]
    struct Ctx { int seg, row0, nrows, n0; const uint8_t* r; };
    __device__ int m_tiles() const { return seg.count(); }
    __device__ bool tile(int bx, int by, Ctx& c) const {
        if (bx >= seg.count()) return false;
        const Tile t = seg.at(bx);
        c.seg = t.seg;
        c.row0 = t.row0;
        c.nrows = t.nrows;
        c.r = experts + (size_t)t.seg * rec;
        c.n0 = by * S::kBN;
        return c.n0 < L;
    }
    __device__ int k_stages(const Ctx&) const { return F / 128; }
    __device__ const uint8_t* a_base(const Ctx& c) const { return h8 + (size_t)c.row0 * F; }
    __device__ const uint8_t* b_base(const Ctx& c) const { return c.r; }
    __device__ uint32_t src_a(const Ctx& c, int i, int lane) const {
        const int r = min(rowmajor_row(i, lane), c.nrows - 1);
        return rowmajor_off((uint32_t)r * F, i, lane);
    }
    // residual: copy i takes rows 16 i .. 16 i + 15 (as MxUp's)
    __device__ const uint8_t* lo_base(const Ctx& c) const { return h4 + (size_t)c.row0 * (F / 2); }
    __device__ uint32_t src_lo(const Ctx& c, int i, int lane) const {
        return (uint32_t)min(16 * i + (lane & 15), c.nrows - 1) * (F / 2) + (lane >> 4) * 16;
    }
    __device__ int b_nb(const Ctx& c, int b) const { return min(c.n0 + b * 16, L - 16) >> 4; }
    __device__ uint32_t src_b(const Ctx& c, int i, int lane) const {
        return (uint32_t)((size_t)F * L + (size_t)b_nb(c, i) * 8 * F) + lane * 16;
    }
    __device__ void scale_src(const Ctx& c, int wave, int lane, const uint8_t*& base, uint32_t& off, int& step) const {
        if (wave == S::kSAW) {
            base = c.r;
            off = (uint32_t)((size_t)3 * F * L / 2 + (size_t)2 * F * L / 32 + (size_t)b_nb(c, lane >> 2) * (F / 2)) +
                  (lane & 3) * 16;
            step = kMxSBStep;
        } else if (S::kLo && wave > S::kSAW && wave < S::kSW) {  // residual scales of rows 64 w + lane
            const int w = wave - S::kSAW - 1;
            base = h4s;
            off = (uint32_t)(c.row0 + min(w * 64 + lane, c.nrows - 1)) * (F / 32);
            step = kMxSAStep;
        } else {  // A scales of rows 64 w + lane (waves past the scale waves copy none; any valid source)
            const int w = wave < S::kSAW ? wave : 0;
            base = h8s;
            off = (uint32_t)(c.row0 + min(w * 64 + lane, c.nrows - 1)) * (F / 32);
            step = kMxSAStep;
        }
    }
    // destination rows of the tile: in registers, or (with the residual operand, whose fragments
    // leave no registers for them) in LDS, written before the barrier that precedes the stores
    static constexpr bool kPrepLds = S::kLo;
    __device__ static int* prep_rows() {
        __shared__ int rows[S::kBM];
        return rows;
    }
    template <int MB>
    struct PrepT {
        int drow[kPrepLds ? 1 : MB][16];
    };
    template <int MB>
    __device__ __forceinline__ PrepT<MB> prep(const Ctx& c, int rb, int lane) const {
        PrepT<MB> q;
        if constexpr (kPrepLds) {
            int* rows = prep_rows();
            for (int m = threadIdx.x; m < S::kBM; m += S::kThreads)
                rows[m] = m < c.nrows ? seg.dest_of(c.seg, c.row0 + m) : -1;
        } else {
#pragma unroll
            for (int i = 0; i < MB; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = rb + i * 32 + frag32_row(r, lane);
                    q.drow[i][r] = m < c.nrows ? seg.dest_of(c.seg, c.row0 + m) : -1;
                }
        }
        return q;
    }
    template <int MB, int NB>
    __device__ __forceinline__ void store(const Ctx& c, f32x16 (&acc)[MB][NB], const PrepT<MB>& q, int rb, int cb,
                                          int lane) const {
        static_for<MB>([&](auto i) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int drow = kPrepLds ? prep_rows()[rb + i * 32 + frag32_row(r, lane)] : q.drow[kPrepLds ? 0 : i][r];
                if (drow >= 0) {
                    const size_t dst = (size_t)drow * L;
                    static_for<NB>([&](auto j) {
                        const int n = c.n0 + cb + j * 32 + frag32_col(lane);
                        if (n < L) Y[dst + n] = (uint16_t)f2bf(acc[i][j][r]);
                    });
                }
            }
        });
    }
};

}  // namespace lmoe
