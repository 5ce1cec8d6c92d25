// Host-side launch wrappers of the latent-MoE kernels (enqueue only; no allocation, no sync).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

namespace lmoe {

struct Tile;

// Outputs of the routing of a batch (each may be null): ids/w [T][k], offsets [E+1], perm/inv
// [T*k], the tile work list and its length, and rowinfo [T*k] = (token, weight bits) of the slot
// at each permuted position ((-1, 0) if none).
struct RouteOut {
    int32_t* ids;
    float* w;
    int32_t* offsets;
    int32_t* perm;
    int32_t* inv;
    Tile* tiles;
    int32_t* ntiles;
    int2* rowinfo;
};

// Optional per-stage event records (the lmoe_forward_opts.stage_events hook).
struct StageEvents {
    void* const* ev;
    hipStream_t s;
    bool capturing = false;
    hipError_t err = hipSuccess;
    StageEvents(void* const* events, hipStream_t stream) : ev(events), s(stream) {
        if (ev) {
            hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
            if (hipStreamIsCapturing(s, &cs) == hipSuccess) capturing = cs == hipStreamCaptureStatusActive;
        }
    }
    // Timing events are not recorded while the stream is being captured: this HIP runtime
    // rejects event-record nodes for timing events inside a capture.
    void rec(int i) {
        if (!ev || !ev[i] || capturing) return;
        const hipError_t r = hipEventRecord(static_cast<hipEvent_t>(ev[i]), s);
        if (r != hipSuccess && err == hipSuccess) err = r;
    }
    void begin(int stage) { rec(2 * stage); }
    void end(int stage) { rec(2 * stage + 1); }
    // the stage's events for a launch that records them itself (hipExtLaunchKernelGGL: the
    // timestamps bracket the kernel's execution, not the dispatch before it); null when not timing
    hipEvent_t start(int stage) const { return ev && !capturing ? static_cast<hipEvent_t>(ev[2 * stage]) : nullptr; }
    hipEvent_t stop(int stage) const { return ev && !capturing ? static_cast<hipEvent_t>(ev[2 * stage + 1]) : nullptr; }
};
constexpr int kStageUp = 5, kStageDown = 6, kStageCombine = 7;  // LMOE_STAGE_EXPERT_UP / _DOWN / COMBINE

// Batches of at most this many tokens use the weight-streaming (decode) kernels.
constexpr int kStreamMaxT = 16;
// Batches of at most this many tokens take the small-batch expert path (two streaming launches)
// and, with a folded router, the small-batch projections.
constexpr int kDecodeMaxT = 64;

#ifndef LMOE_ROUTE_IN_EXPERTS
#define LMOE_ROUTE_IN_EXPERTS 1
#endif
// Small batches: route inside the gate/up launch (one dependent launch fewer).
constexpr bool kRouteInExperts = LMOE_ROUTE_IN_EXPERTS != 0;

hipError_t launch_rmsnorm(const float* h, int T, int H, uint16_t* x16, hipStream_t s);

// mode 0: out32 = xW^T and out16 = bf16(out32); 1: out16 = bf16(xW^T); 2: out32 += xW^T
// (mode 0, T > kStreamMaxT: out32 may be null, then only the bf16 outputs are written)
// out16lo (mode 0, T > kStreamMaxT, optional): also write the low bf16 half of the output.
// out16h (mode 0, small batches, optional): also write fp16 of the output.
// hnorm (small batches staged in LDS only, i.e. T <= kStreamMaxT and small_proj_fits): the input
// is bf16(RMSNorm(hnorm)) of an fp32 residual [T][K] (unit gain, eps 1e-6) instead of x.
hipError_t launch_proj_bf16(const uint16_t* x, const uint16_t* W, int T, int N, int K, int mode, float* out32,
                            uint16_t* out16, hipStream_t s, uint16_t* out16lo = nullptr, uint16_t* out16h = nullptr,
                            const float* hnorm = nullptr);

// zhi/zlo (T > kStreamMaxT, optional): the bf16 halves of z written by the D projection; then
// logits holds [2][T][E]: the hi half's logits (+ br) and the lo half's, which the top-k adds.
hipError_t launch_router_bf16(const float* z, const uint16_t* Wr, const float* br, int T, int E, int L, float* logits,
                              hipStream_t s, const uint16_t* zhi = nullptr, const uint16_t* zlo = nullptr);

// logits2 (optional): a second [T][E] half added to logits.
hipError_t launch_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w, hipStream_t s,
                       const float* logits2 = nullptr);

// logits [2][T][E] of a batch from x [T][K] bf16 and the folded router Gr [E][2][K]: half h is
// x . Gr[e][h], br (optional) added to half 0.
hipError_t launch_router_x(const uint16_t* x, const uint16_t* Gr, const float* br, int T, int E, int K, float* logits,
                           hipStream_t s);


int perm_blocks(int T);

// tiles may be null (no work list).  hist/base: [perm_blocks(T)][E] ints (unused when T <= 64):
// per block of 64 tokens, each expert's slot count, and its inclusive running count.
hipError_t launch_permute(const int32_t* ids, int T, int k, int E, int32_t* hist, int32_t* base, int32_t* offsets,
                          int32_t* perm, int32_t* inv, int BM, Tile* tiles, int32_t* ntiles, int has_shared,
                          hipStream_t s);

// top-k followed by the permutation; one fused launch when T <= 64.  logits2 (optional): a
// second [T][E] half added to logits (the folded router's lo half).  rowinfo (T <= 64
// only): [T*k] (token, weight bits) of the slot at each permuted position, (-1, 0) if none.
hipError_t launch_topk_permute(const float* logits, int T, int E, int k, int32_t* ids, float* w, int32_t* hist,
                               int32_t* base, int32_t* offsets, int32_t* perm, int32_t* inv, int BM, Tile* tiles,
                               int32_t* ntiles, int has_shared, hipStream_t s, const float* logits2 = nullptr,
                               int2* rowinfo = nullptr);

// Whether a batch takes the small-batch expert path (gate/up launch, down + merge launch into
// decode_groups() partial merged rows, summed by the U projection).
bool decode_fits(int T, int L, int F, int Fs);
// Whether a T-token projection with reduction width K stages its input in LDS (one launch).
bool small_proj_fits(int T, int K);
int decode_groups();

// Small batch: z = x D^T (z32 and bf16 z16) and the folded router's logits in one launch:
// logits [2][T][E], logits[0] = x hi^T + br, logits[1] = x lo^T (the top-k adds them).
// hnorm (optional): x is bf16(RMSNorm(hnorm)) of an fp32 residual [T][H], formed while staging.
hipError_t launch_proj_router_bf16(const uint16_t* x, const uint16_t* D, const uint16_t* Gr, const float* br, int T,
                                  int L, int H, int E, float* z32, uint16_t* z16, float* logits, hipStream_t s,
                                  uint16_t* z16h = nullptr, const float* hnorm = nullptr);
// Gr [E][2][H] = hi and lo bf16 halves of Wr . D (fp32 accumulation); with expert groups of Eg
// experts, row e uses D rows (e / Eg) * L .. (Eg = 0: one group).
hipError_t launch_fold_router(const uint16_t* D, const uint16_t* Wr, int E, int L, int H, uint16_t* Gr, hipStream_t s,
                              int Eg = 0);

// U projection of a small batch with expert groups: input rows of KG * K columns, the sum (in
// order, in fp32) of G bf16 partials [G][T][KG * K]; one launch multiplies each K group into part
// [KG][T][N] fp32, a second sums the groups in order (mode 1: bf16 out16; 2: out32 +=).
hipError_t launch_proj_partials_kgroups(const uint16_t* xpart, int G, const uint16_t* W, int T, int N, int K, int KG,
                                        float* part, int mode, float* out32, uint16_t* out16, hipStream_t s);

// U projection of a small batch whose input is the sum (in order, in fp32) of G bf16 partials [G][T][K].
hipError_t launch_proj_partials(const uint16_t* xpart, int G, const uint16_t* W, int T, int N, int K, int mode, float* out32,
                                uint16_t* out16, hipStream_t s);

// Rows of the expert work list's tiles: 16 (small batches), 128 (the block-scaled MXFP4 kernels),
// else the rows of the large-batch bf16 GEMM tiles (256).
int expert_tile_rows(bool stream_path, bool mx_path, int T, int k, int E);
int expert_max_tiles(int T, int k, int E, int has_shared, bool stream_path, bool mx_path);

// Routing done inside the small-batch gate/up launch (T <= 64): the logits (hi half, and the lo
// half of a folded router or null) and where the routing outputs go.
struct ExpertRoute {
    const float* logits;
    const float* logits2;
    int BM, has_shared;
    RouteOut out;
};

struct ExpertArgs {
    const Tile* tiles;
    const int32_t* ntiles;
    const int32_t* perm;
    int T, k, E, L, F, Fs, Hs;
    const uint16_t* z16;
    const uint16_t* z16h;  // fp16 copy of z16 or null (4-bit experts convert z16 themselves)
    const void* experts;
    size_t rec_bytes;
    const void* shared;
    uint16_t* H;
    uint16_t* Y;       // [T*k + T][L] bf16 expert outputs (larger batches)
    int max_tiles;
    bool stream_path;
    bool decode_path;  // small batch: gate/up into H, then down + merge into mpart
    int fmt;           // routed expert records: 0 bf16, 1 MXFP4, 2 NVFP4
    uint16_t* mpart;   // [decode_groups()][T][zp] partial merged rows in bf16 (decode path)
    const float* w;
    const int2* rowinfo;  // decode path: [T*k] (token, weight bits) per permuted position
    const ExpertRoute* route;  // decode path: non-null = route inside the gate/up launch
    int Eg = 0;  // experts per expert group (0: one group)
    int zp = 0;  // row pitch of z16 / z16h / mpart: L times the expert groups (0: L)
    // 4-bit records on the tile path (large batches): decoded bf16 records [E][3 F L] and the
    // records' tensor scales [E][3]; offsets [E + 1] says which experts have tokens
    uint16_t* deq = nullptr;
    float* deq_ts = nullptr;
    const int32_t* offsets = nullptr;
    // MXFP4 records on the block-scaled MFMA path (large batches): z as MXFP8 [T][zp] values and
    // [T][zp / 32] scales plus its MXFP4 residual [T][zp / 2] and [T][zp / 32], the routed rows of
    // H in bf16 [T k][F], then as MXFP8 [T k][F] and [T k][F / 32] plus its MXFP4 residual
    // [T k][F / 2] and [T k][F / 32]
    bool mx_path = false;
    uint8_t* z8 = nullptr;
    uint8_t* z8s = nullptr;
    uint8_t* z4 = nullptr;
    uint8_t* z4s = nullptr;
    uint8_t* h8 = nullptr;
    uint8_t* h8s = nullptr;
    uint8_t* h4 = nullptr;
    uint8_t* h4s = nullptr;
    uint16_t* h16 = nullptr;
    int tile_rows = 0;  // rows of the work list's tiles (expert_tile_rows)
};

// Large 4-bit batches: minimum T at which the records of the experts with tokens are decoded to
// bf16 once and the bf16 tile GEMMs run (below it the weight-streaming kernels read the 4-bit
// records directly).  Measured at the 145B shape with MXFP4 records: streaming is faster at
// T = 256 (542 vs 580 us), decoding at T = 512 (655 vs 795 us) and beyond.
#ifndef LMOE_DEQUANT_MIN_T
#define LMOE_DEQUANT_MIN_T 384
#endif
constexpr int kDequantMinT = LMOE_DEQUANT_MIN_T;
// MXFP4 layers: minimum T of the block-scaled MFMA path (no record decode, so it pays off earlier).
// Measured at the 145B shape (us per layer, weight-streaming kernels vs this path): T = 96 362 vs
// 338, 128 423 vs 352, 192 497 vs 424, 256 580 vs 442, 320 630 vs 456.
#ifndef LMOE_MX_MIN_T
#define LMOE_MX_MIN_T 96
#endif
constexpr int kMxMinT = LMOE_MX_MIN_T;
hipError_t launch_experts_bf16(const ExpertArgs& a, hipStream_t s, StageEvents& ev);

// Row-major expert records -> packed records (nrec records of rec_bytes; F x L gate/up, L x F down;
// fmt 0 bf16, 1 MXFP4, 2 NVFP4).
hipError_t launch_pack(const void* src, void* dst, size_t rec_bytes, int nrec, int F, int L, int fmt, hipStream_t s);

// Y: bf16 rows when out_bf16 (the bf16 path), else fp32 rows.  With expert groups (groups > 1,
// Eg experts each, ids [T][k]) m is [T][groups * L], group g's merged row in columns g * L ..
hipError_t launch_combine(const void* Y, const float* w, int T, int k, int L, int has_shared, bool out_bf16, void* m,
                          hipStream_t s, const int32_t* ids = nullptr, int groups = 1, int Eg = 0);

// fp32 path. mode 0: out = xW^T (+bias); 2: out += xW^T
hipError_t launch_proj_f32(const float* x, const float* W, const float* bias, int T, int N, int K, int mode, float* out,
                           hipStream_t s);

struct F32ExpertArgs {
    const float* z;
    const int32_t* ids;
    const int32_t* perm;
    const float* experts;
    const float* shared;
    int T, k, L, F, Fs, Hs;
    float* H;
    float* Y;
};
hipError_t launch_experts_f32(const F32ExpertArgs& a, hipStream_t s, StageEvents& ev);

}  // namespace lmoe
