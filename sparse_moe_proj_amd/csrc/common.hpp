// Shared device definitions for the latent-MoE kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <type_traits>

namespace lmoe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

// ----------------------------------------------------------------------------------------------
// scalar conversions
// ----------------------------------------------------------------------------------------------
__device__ __forceinline__ float bf2f(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// float -> bf16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t f2bf(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) { return f2bf(lo) | (f2bf(hi) << 16); }
// a[0..7] += the 8 bf16 values of u (low half of each dword first)
__device__ __forceinline__ void add_bf16x8(float (&a)[8], const uint4& u) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a[2 * i] += bf2f(w[i] & 0xFFFFu);
        a[2 * i + 1] += bf2f(w[i] >> 16);
    }
}

// v through an opaque move (a VGPR copy the compiler cannot see through): values computed from
// it are recomputed where they are used, not hoisted out of a kernel's outer loop and kept (or
// spilled) across it.
__device__ __forceinline__ int opaque(int v) {
    int r;
    __asm__ volatile("v_mov_b32 %0, %1" : "=v"(r) : "v"(v));
    return r;
}

// SiLU with the hardware reciprocal (v_rcp_f32, about 1 ulp): x / (1 + e^-x) as x * rcp(1 + e^-x).
// Large negative x give e^-x = inf, rcp(inf) = 0 and a zero result.
__device__ __forceinline__ float silu(float v) { return v * __builtin_amdgcn_rcpf(1.0f + __expf(-v)); }

// bf16 of f, rounded to nearest even by gfx950's conversion instruction (v_cvt_pk_bf16_f32), for
// values that are only stored (the routing inputs keep the integer rounding of f2bf).
__device__ __forceinline__ uint16_t bf16_rn(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
__device__ __forceinline__ uint32_t pack_bf2_rn(float lo, float hi) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// 16 bytes reinterpreted as 8 bf16 MFMA operands.
__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// Split an fp32 value into hi = bf16(v) and lo = bf16(v - hi); hi + lo carries ~16 significand
// bits, enough for router logits that must stay within ~1e-5 of their fp32 value.
__device__ __forceinline__ void split_hi_lo(float v, uint32_t& hi, uint32_t& lo) {
    hi = f2bf(v);
    lo = f2bf(v - bf2f(hi));
}

// ----------------------------------------------------------------------------------------------
// MFMA wrappers (CDNA4 dense bf16, fp32 accumulate)
//   32x32x16: A lane l holds row (l%32), k = 8*(l/32)+0..7; B lane l holds col (l%32), same k;
//             D register r of lane l is row 8*(r/4) + 4*(l/32) + (r%4), col l%32.
//   16x16x32: A lane l holds row (l%16), k = 8*(l/16)+0..7; B lane l holds col (l%16), same k;
//             D register r of lane l is row 4*(l/16) + r, col l%16.
// ----------------------------------------------------------------------------------------------
__device__ __forceinline__ f32x16 mfma32(uint4 a, uint4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(uint4 a, uint4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}
// The same shape with fp16 operands (the 4-bit expert rows decode to fp16).
__device__ __forceinline__ f32x4 mfma16_f16(uint4 a, uint4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// ----------------------------------------------------------------------------------------------
// 4-bit decoding: 8 E2M1 nibbles (one 32-bit word, low nibble first) times a block scale
// -> 8 bf16 values (16 bytes, the layout of one MFMA operand).  An E2M1 magnitude has at most
// two significant bits and both block scales (a power of two; an E4M3 value, at most four
// significant bits) multiply it exactly, so the bf16 operands are the exact decoded values.
// ----------------------------------------------------------------------------------------------
__device__ __forceinline__ uint4 fp4x8_to_bf16x8(uint32_t nib8, float scale) {
    uint32_t out[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t n0 = (nib8 >> (8 * i)) & 0xFu;
        uint32_t n1 = (nib8 >> (8 * i + 4)) & 0xFu;
        // E2M1 magnitudes as fp32 from the code: code c = e*2 + m (e: 2-bit exponent, m: mantissa);
        // by code: 0, 0.5, 1, 1.5, 2, 3, 4, 6
        auto mag = [](uint32_t c) -> float {
            uint32_t e = (c >> 1) & 3u, m = c & 1u;
            // e == 0: subnormal m * 0.5; else (1 + m/2) * 2^(e-1)
            return e == 0 ? 0.5f * (float)m : __uint_as_float(((126u + e) << 23) | (m << 22));
        };
        float v0 = mag(n0) * scale;
        float v1 = mag(n1) * scale;
        v0 = (n0 & 8u) ? -v0 : v0;
        v1 = (n1 & 8u) ? -v1 : v1;
        out[i] = pack_bf2(v0, v1);
    }
    return make_uint4(out[0], out[1], out[2], out[3]);
}

// MXFP4 block scale: E8M0 byte s -> 2^(s - 127) (byte 0 is 2^-127, a float32 subnormal).
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) { return __uint_as_float(s == 0 ? 0x00400000u : (s << 23)); }

// NVFP4 block scale: FP8 E4M3 byte (sign, 4 exponent bits with bias 7, 3 mantissa bits; exponent
// 0 subnormal, m/8 * 2^-6) -> float32, exactly.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
    const uint32_t e = (b >> 3) & 0xFu, m = b & 7u;
    const float mag = e == 0 ? (float)m * 0.001953125f /* 2^-9 */ : __uint_as_float(((e + 120u) << 23) | (m << 20));
    return (b & 0x80u) ? -mag : mag;
}

__device__ __forceinline__ uint4 mxfp4_to_bf16x8(uint32_t nib8, uint32_t scale_byte) {
    return fp4x8_to_bf16x8(nib8, e8m0_to_f32(scale_byte));
}

// 8 E2M1 nibbles (value i in bits 4i .. 4i + 3) -> 8 fp16 values (pairs in value order) times a
// power of two, by gfx950's conversion instruction (one per byte: the lower nibble becomes the
// low half).  The instruction applies only the exponent of its fp32 scale operand, so `pow2` must
// be a power of two (an E8M0 block scale); the results are then exact, fp16 subnormals included
// (checked against a table of every byte value, scales 2^-15 .. 1).
__device__ __forceinline__ uint4 fp4x8_to_f16x8_pow2(uint32_t w, float pow2) {
    return make_uint4(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, pow2, 0)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, pow2, 1)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, pow2, 2)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, pow2, 3)));
}

// 8 E2M1 nibbles -> 8 fp16 values times any block scale (fp16 pair `scale2`, both halves equal):
// the exact fp16 E2M1 values, then one packed fp16 multiply per pair.
__device__ __forceinline__ uint4 fp4x8_to_f16x8(uint32_t w, uint32_t scale2) {
    const uint4 v = fp4x8_to_f16x8_pow2(w, 1.f);
    const f16x2 sc = __builtin_bit_cast(f16x2, scale2);
    uint32_t o[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, o[i]) * sc);
    return make_uint4(o[0], o[1], o[2], o[3]);
}

// fp16 pair (v, v) of a float (round to nearest even).
__device__ __forceinline__ uint32_t f16x2_splat(float v) {
    const _Float16 h = (_Float16)v;
    return __builtin_bit_cast(uint32_t, f16x2{h, h});
}

// Two FP8 E4M3 bytes (bits 0-7 and 8-15 of b) -> an fp16 pair, exactly.  An E4M3 byte's
// exponent and mantissa fields, moved into an fp16's (sign to bit 15, the 7 other bits to bits
// 7..13), read as an fp16 whose exponent bias is 15 instead of 7, i.e. 2^-8 times the E4M3 value
// (its subnormals land on fp16 subnormals the same way); one packed multiply by 256 restores it.
__device__ __forceinline__ uint32_t e4m3x2_to_f16x2(uint32_t b) {
    const uint32_t u = (b & 0xFFu) | ((b & 0xFF00u) << 8);  // byte 0 at bits 0-7, byte 1 at 16-23
    const uint32_t h = ((u & 0x007F007Fu) << 7) | ((u & 0x00800080u) << 8);
    const _Float16 k = (_Float16)256.0f;
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, h) * f16x2{k, k});
}

// float -> fp16 (round to nearest even), magnitudes beyond the largest finite fp16 (65504)
// saturating to it instead of becoming infinities.  The 4-bit small-batch kernels carry z and
// the SwiGLU rows in fp16; activations past that range lose their size but stay finite.
__device__ __forceinline__ _Float16 f16_sat(float v) { return (_Float16)fminf(fmaxf(v, -65504.f), 65504.f); }

// 8 bf16 -> 8 fp16 (exact for values in fp16's normal range; saturating beyond it).
__device__ __forceinline__ uint4 bf16x8_to_f16x8(uint4 v) {
    uint32_t o[4];
    const uint32_t in[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
        o[i] = __builtin_bit_cast(uint32_t, f16x2{f16_sat(__uint_as_float(in[i] << 16)),
                                                  f16_sat(__uint_as_float(in[i] & 0xFFFF0000u))});
    return make_uint4(o[0], o[1], o[2], o[3]);
}

// fp32 pair -> fp16 pair bits (round to nearest even, saturating).
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, f16x2{f16_sat(lo), f16_sat(hi)});
}

// ----------------------------------------------------------------------------------------------
// work lists
// ----------------------------------------------------------------------------------------------
// One tile of a grouped GEMM: `seg` is the expert id (n_experts = the shared expert),
// rows [row0, row0 + nrows) of the segment-ordered row space.
struct Tile {
    int32_t seg;
    int32_t row0;
    int32_t nrows;
    int32_t pad;
};

// Logical tile of this workgroup.  The grid is (N tiles, M tiles); workgroups are handed to the
// 8 XCDs round-robin, so the linear id is remapped to give each XCD a contiguous run of logical
// tiles: the N tiles of one M tile (sharing its activation rows) then run on one XCD, one after
// the other, and its L2 serves the shared operand.
__device__ __forceinline__ void xcd_tile(int& m_tile, int& n_tile) {
    const int total = gridDim.x * gridDim.y;
    const int bid = blockIdx.x + gridDim.x * blockIdx.y;
    const int per = total / 8, rem = total % 8;
    const int x = bid % 8, i = bid / 8;
    const int l = x * per + min(x, rem) + i;
    n_tile = l % gridDim.x;
    m_tile = l / gridDim.x;
}

// A type carried as a value (to pick a template argument from a generic lambda).
template <class T>
struct TypeTag {
    using type = T;
};

// Calls f(integral_constant<int, I>) for I = 0 .. N-1 (compile-time indices, so register arrays
// indexed with them stay in registers however large the unrolled body gets).
template <int N, int I = 0, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<N, I + 1>(static_cast<F&&>(f));
    }
}

}  // namespace lmoe
