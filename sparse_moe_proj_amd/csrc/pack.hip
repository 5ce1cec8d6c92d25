// Re-layout of expert records from row-major matrices into the packed tile order the expert
// kernels read (see packed_row in problems.hpp): a pure permutation of 16-byte units (and of
// scale units for the 4-bit formats), record by record.
#include "launch.hpp"

namespace lmoe {
namespace {

// Position of unit c of row n in a packed matrix with `upr` units per row; four units make one
// column step (bf16: 4 x 8 columns; MXFP4 nibbles or scales: 4 x 32 values).
__device__ __forceinline__ size_t packed_unit(int n, int c, int upr) {
    return ((size_t)(n >> 4) * (upr >> 2) + (c >> 2)) * 64 + (c & 3) * 16 + (n & 15);
}

// One matrix [N][upr units of UB bytes] at byte offset `off` of every record (blockIdx.y).
template <int UB>
__global__ __launch_bounds__(256) void pack_matrix_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                          size_t rec_bytes, size_t off, int N, int upr) {
    const size_t u = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
    if (u >= (size_t)N * upr) return;
    const int n = (int)(u / upr), c = (int)(u % upr);
    const size_t base = blockIdx.y * rec_bytes + off;
    const uint8_t* s = src + base + u * UB;
    uint8_t* d = dst + base + packed_unit(n, c, upr) * UB;
    if constexpr (UB == 16)
        *reinterpret_cast<uint4*>(d) = *reinterpret_cast<const uint4*>(s);
    else if constexpr (UB == 2)
        *reinterpret_cast<uint16_t*>(d) = *reinterpret_cast<const uint16_t*>(s);
    else
        *d = *s;
}

template <int UB>
hipError_t pack_matrix(const uint8_t* src, uint8_t* dst, size_t rec_bytes, int nrec, size_t off, int N, int upr,
                       hipStream_t s) {
    const size_t units = (size_t)N * upr;
    hipLaunchKernelGGL(pack_matrix_kernel<UB>, dim3((unsigned)((units + 255) / 256), nrec), dim3(256), 0, s, src, dst,
                       rec_bytes, off, N, upr);
    return hipGetLastError();
}

}  // namespace

// Records of F x L gate/up and L x F down matrices; fmt 0: bf16; 1: MXFP4 nibbles then E8M0 scales
// (one byte per 32 values); 2: NVFP4 nibbles, E4M3 scales (one byte per 16 values, moved as
// 2-byte units: the two blocks of a 32-value unit), then the three fp32 tensor scales (copied).
hipError_t launch_pack(const void* src, void* dst, size_t rec_bytes, int nrec, int F, int L, int fmt, hipStream_t s) {
    const uint8_t* a = static_cast<const uint8_t*>(src);
    uint8_t* b = static_cast<uint8_t*>(dst);
    const size_t fl = (size_t)F * L;
    hipError_t e;
    if (fmt == 2) {
        const size_t nb = fl / 2, sb = fl / 16;
        if ((e = pack_matrix<16>(a, b, rec_bytes, nrec, 0, F, L / 32, s)) != hipSuccess) return e;
        if ((e = pack_matrix<16>(a, b, rec_bytes, nrec, nb, F, L / 32, s)) != hipSuccess) return e;
        if ((e = pack_matrix<16>(a, b, rec_bytes, nrec, 2 * nb, L, F / 32, s)) != hipSuccess) return e;
        if ((e = pack_matrix<2>(a, b, rec_bytes, nrec, 3 * nb, F, L / 32, s)) != hipSuccess) return e;
        if ((e = pack_matrix<2>(a, b, rec_bytes, nrec, 3 * nb + sb, F, L / 32, s)) != hipSuccess) return e;
        if ((e = pack_matrix<2>(a, b, rec_bytes, nrec, 3 * nb + 2 * sb, L, F / 32, s)) != hipSuccess) return e;
        return pack_matrix<16>(a, b, rec_bytes, nrec, 3 * nb + 3 * sb, 1, 1, s);  // tensor scales: one unit
    }
    if (fmt == 0) {
        if ((e = pack_matrix<16>(a, b, rec_bytes, nrec, 0, F, L / 8, s)) != hipSuccess) return e;
        if ((e = pack_matrix<16>(a, b, rec_bytes, nrec, fl * 2, F, L / 8, s)) != hipSuccess) return e;
        return pack_matrix<16>(a, b, rec_bytes, nrec, 2 * fl * 2, L, F / 8, s);
    }
    const size_t nb = fl / 2, sb = fl / 32;
    if ((e = pack_matrix<16>(a, b, rec_bytes, nrec, 0, F, L / 32, s)) != hipSuccess) return e;
    if ((e = pack_matrix<16>(a, b, rec_bytes, nrec, nb, F, L / 32, s)) != hipSuccess) return e;
    if ((e = pack_matrix<16>(a, b, rec_bytes, nrec, 2 * nb, L, F / 32, s)) != hipSuccess) return e;
    if ((e = pack_matrix<1>(a, b, rec_bytes, nrec, 3 * nb, F, L / 32, s)) != hipSuccess) return e;
    if ((e = pack_matrix<1>(a, b, rec_bytes, nrec, 3 * nb + sb, F, L / 32, s)) != hipSuccess) return e;
    return pack_matrix<1>(a, b, rec_bytes, nrec, 3 * nb + 2 * sb, L, F / 32, s);
}

}  // namespace lmoe
