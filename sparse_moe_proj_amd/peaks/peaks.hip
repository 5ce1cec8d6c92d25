// Measurement kernels for the benchmark, kept out of the block's library: the HBM read rate a
// plain streaming kernel reaches on this part, the issue rate of back-to-back matrix-core
// instructions (bf16 32x32x16 and the block-scaled FP8 x FP4 32x32x64), and the shader clock
// while they run.  They compute nothing of the block; bench.py reports the block's kernels
// against these measured rates beside the published peaks.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// Every thread reads 16-byte units i, i + stride, ... (four in flight per iteration) and folds
// them into one word, written only if it equals a value no input of the benchmark produces, so
// the loads stay and nothing else touches memory.
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* __restrict__ p, size_t n, uint32_t* sink) {
    const size_t stride = (size_t)gridDim.x * 256;
    size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 3 * stride < n; i += 4 * stride) {
        const uint4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
        acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
    }
    for (; i < n; i += stride) {
        const uint4 a = p[i];
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

// Shader-clock and 100 MHz real-time counters at the start and end of wave 0 of workgroup 0.
__device__ __forceinline__ void stamp(unsigned long long* clk, int at) {
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        clk[2 * at] = __builtin_amdgcn_s_memtime();
        clk[2 * at + 1] = __builtin_amdgcn_s_memrealtime();
    }
}

// NACC independent accumulators per wave, `iters` rounds of one MFMA each; operands from the
// thread index (not constants), the sums written so that nothing is dropped.
constexpr int kAcc = 8;

__global__ __launch_bounds__(256) void mfma_bf16_kernel(float* out, int iters, unsigned long long* clk) {
    f32x16 acc[kAcc];
#pragma unroll
    for (int u = 0; u < kAcc; ++u) acc[u] = f32x16{};
    const float s = (float)(threadIdx.x & 7) * 0.125f;
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)(s + e);
        b[e] = (__bf16)(s - e);
    }
    stamp(clk, 0);
    for (int i = 0; i < iters; ++i)
#pragma unroll
        for (int u = 0; u < kAcc; ++u) acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[u], 0, 0, 0);
    stamp(clk, 1);
    float t = 0.f;
#pragma unroll
    for (int u = 0; u < kAcc; ++u)
#pragma unroll
        for (int r = 0; r < 16; ++r) t += acc[u][r];
    out[(size_t)blockIdx.x * 256 + threadIdx.x] = t;
}

// v_mfma_scale_f32_32x32x64_f8f6f4 with an FP8 E4M3 A operand and an FP4 E2M1 B operand (the
// form of the MXFP4 expert products), unit E8M0 scales (byte 127).
__global__ __launch_bounds__(256) void mfma_fp8fp4_kernel(float* out, int iters, unsigned long long* clk) {
    f32x16 acc[kAcc];
#pragma unroll
    for (int u = 0; u < kAcc; ++u) acc[u] = f32x16{};
    const int s = (int)(threadIdx.x & 7);
    i32x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = 0x38383838 + s;  // E4M3 bytes near 1.0
        b[e] = e < 4 ? 0x22222222 + s : 0;  // E2M1 nibbles of 1.0 (the FP4 operand is 16 bytes)
    }
    stamp(clk, 0);
    for (int i = 0; i < iters; ++i)
#pragma unroll
        for (int u = 0; u < kAcc; ++u)
            acc[u] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[u], 0, 4, 0, 127, 0, 127);
    stamp(clk, 1);
    float t = 0.f;
#pragma unroll
    for (int u = 0; u < kAcc; ++u)
#pragma unroll
        for (int r = 0; r < 16; ++r) t += acc[u][r];
    out[(size_t)blockIdx.x * 256 + threadIdx.x] = t;
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16) of `buf` with `grid` workgroups of 256 threads; sink holds
// `grid` words.
int peak_stream_read(const void* buf, size_t bytes, uint32_t* sink, int grid, void* stream) {
    hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint4*>(buf), bytes / 16, sink);
    return (int)hipGetLastError();
}

// `grid` workgroups of 4 waves (one per SIMD of a CU), each wave `iters` x 8 MFMAs; out holds
// grid * 256 floats, clk 4 words (shader clock and real time at the start and the end).
// kind 0: bf16 32x32x16 (32768 flop each); 1: scaled FP8 x FP4 32x32x64 (131072 flop each).
int peak_mfma(int kind, float* out, int iters, unsigned long long* clk, int grid, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (kind == 0)
        hipLaunchKernelGGL(mfma_bf16_kernel, dim3(grid), dim3(256), 0, s, out, iters, clk);
    else
        hipLaunchKernelGGL(mfma_fp8fp4_kernel, dim3(grid), dim3(256), 0, s, out, iters, clk);
    return (int)hipGetLastError();
}

int peak_mfma_per_wave() { return kAcc; }

}  // extern "C"
