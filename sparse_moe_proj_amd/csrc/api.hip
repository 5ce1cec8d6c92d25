// C ABI of the latent-MoE block: argument validation, workspace layout and launch order.
// Everything here runs on the host and only enqueues work on the caller's stream.
#include <stdarg.h>
#include <stdio.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <string>

#include "common.hpp"
#include "launch.hpp"
#include "lmoe.h"

using namespace lmoe;

namespace {

thread_local std::string g_err;

lmoe_status fail(lmoe_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

lmoe_status hip_fail(hipError_t e, const char* where) {
    return fail(LMOE_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

struct Dims {
    int H, L, E, k, F, Fs;
    int G, Eg, Lz;  // expert groups, experts per group, z width G * L
    bool f32;  // fp32 storage end to end
    bool mx;   // 4-bit routed experts (MXFP4 or NVFP4)
    int fmt;   // routed expert records: 0 bf16 (or fp32), 1 MXFP4, 2 NVFP4
    int mx_min_t;  // MXFP4: smallest batch of the block-scaled MFMA kernels (INT32_MAX: never)
};

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

lmoe_status check_config(const lmoe_config* cfg, Dims& d) {
    if (!cfg) return fail(LMOE_ERR_NULL, "cfg is NULL");
    const int a = cfg->act_dtype, dn = cfg->dense_dtype, ex = cfg->expert_dtype;
    if (a < 0 || a > 3 || dn < 0 || dn > 3 || ex < 0 || ex > 3) return fail(LMOE_ERR_DTYPE, "unknown dtype code");
    const bool f32 = a == LMOE_F32 && dn == LMOE_F32 && ex == LMOE_F32;
    const bool bf = a == LMOE_BF16 && dn == LMOE_BF16 && (ex == LMOE_BF16 || ex == LMOE_MXFP4 || ex == LMOE_NVFP4);
    if (!f32 && !bf)
        return fail(LMOE_ERR_UNSUPPORTED, "dtype combination act=%d dense=%d expert=%d is not supported", a, dn, ex);
    d.H = cfg->hidden;
    d.L = cfg->latent;
    d.E = cfg->n_experts;
    d.k = cfg->top_k;
    d.F = cfg->ffn;
    d.Fs = cfg->shared_ffn;
    d.f32 = f32;
    d.mx = ex == LMOE_MXFP4 || ex == LMOE_NVFP4;
    d.fmt = ex == LMOE_MXFP4 ? 1 : ex == LMOE_NVFP4 ? 2 : 0;
    if (d.H <= 0 || d.L <= 0 || d.F <= 0 || d.H % 64 || d.L % 64 || d.F % 64)
        return fail(LMOE_ERR_SHAPE, "hidden, latent and ffn must be positive multiples of 64 (got %d, %d, %d)", d.H, d.L,
                    d.F);
    if (d.Fs < 0 || d.Fs % 64) return fail(LMOE_ERR_SHAPE, "shared_ffn must be 0 or a multiple of 64 (got %d)", d.Fs);
    if (d.mx && (d.L % 128 || d.F % 128 || d.Fs % 128))
        return fail(LMOE_ERR_SHAPE, "4-bit experts need latent, ffn and shared_ffn to be multiples of 128");
    if (d.k < 1 || d.k > 16) return fail(LMOE_ERR_SHAPE, "top_k must be in [1, 16] (got %d)", d.k);
    if (d.E < d.k || d.E > 1024) return fail(LMOE_ERR_SHAPE, "n_experts must be in [top_k, 1024] (got %d)", d.E);
    if ((long)d.H * d.L > (1L << 30) || (long)d.F * d.L > (1L << 30) || (long)d.Fs * d.L > (1L << 30))
        return fail(LMOE_ERR_SHAPE, "a weight matrix exceeds 2^30 elements");
    d.G = cfg->groups > 1 ? cfg->groups : 1;
    if (cfg->groups < 0 || d.G > 64 || d.E % d.G)
        return fail(LMOE_ERR_SHAPE, "groups must be in [0, 64] and divide n_experts (got %d)", cfg->groups);
    if (d.G > 1 && f32) return fail(LMOE_ERR_UNSUPPORTED, "expert groups need bf16 activations and dense weights");
    d.Eg = d.E / d.G;
    d.Lz = d.G * d.L;
    if ((long)d.H * d.Lz > (1L << 30)) return fail(LMOE_ERR_SHAPE, "D or U exceeds 2^30 elements");
    if (cfg->mx_mfma_min_t < -1)
        return fail(LMOE_ERR_SHAPE, "mx_mfma_min_t must be -1, 0 or a batch size (got %d)", cfg->mx_mfma_min_t);
    d.mx_min_t = cfg->mx_mfma_min_t < 0 ? INT32_MAX
                                        : std::max(cfg->mx_mfma_min_t == 0 ? kMxMinT : cfg->mx_mfma_min_t, kDecodeMaxT + 1);
    return LMOE_OK;
}

lmoe_status check_T(const Dims& d, int32_t T) {
    if (T < 0 || T > (1 << 20)) return fail(LMOE_ERR_SHAPE, "T must be in [0, 2^20] (got %d)", T);
    if ((long)T * d.k >= (1L << 31) - (1L << 24)) return fail(LMOE_ERR_SHAPE, "T * top_k too large");
    if ((long)T * d.Lz * 2 >= (1L << 32)) return fail(LMOE_ERR_SHAPE, "T * groups * latent too large");
    return LMOE_OK;
}

constexpr size_t kAlign = 256;
size_t up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct Layout {
    size_t x16, z32, z16, z16h, zlo, logits, ids, w, offsets, perm, inv, rowinfo, hist, base, tiles, ntiles, H, Y, mpart, m,
        deq, deq_ts, z8, z8s, z4, z4s, h8, h8s, h4, h4s, h16, total;
    bool stream_path, decode_path, fused_router, deq_path, mx_path;
    int max_tiles, BM, Hs, R;
};

Layout plan(const Dims& d, int T) {
    Layout lo{};
    const size_t act = d.f32 ? 4 : 2;
    const int has_shared = d.Fs > 0;
    lo.decode_path = !d.f32 && decode_fits(T, d.L, d.F, d.Fs);
    // 4-bit records stream through the weight-streaming kernels up to kDequantMinT tokens; larger
    // batches decode the touched records to bf16 once and take the tile GEMMs
    // MXFP4 takes the block-scaled MFMA kernels from d.mx_min_t tokens (never: the decode to bf16
    // from kDequantMinT, as NVFP4)
    lo.mx_path = d.fmt == 1 && !lo.decode_path && T >= d.mx_min_t;
    const bool deq = d.mx && !lo.decode_path && !lo.mx_path && T >= kDequantMinT;
    const bool big4 = lo.mx_path || deq;
    lo.deq_path = deq;
    lo.stream_path = !d.f32 && (T <= kStreamMaxT || (d.mx && !big4) || lo.decode_path);
    lo.fused_router = !d.f32 && small_proj_fits(T, d.H);
    // expert groups take the logits from x and the folded router for every batch, and batches
    // above kStreamMaxT multiply the two bf16 halves of z separately: two halves of logits
    const bool halves = lo.fused_router || d.G > 1 || (!d.f32 && T > kStreamMaxT);
    lo.BM = expert_tile_rows(lo.stream_path, lo.mx_path, T, d.k, d.E);
    lo.max_tiles = expert_max_tiles(T, d.k, d.E, has_shared, lo.stream_path, lo.mx_path);
    lo.Hs = std::max(d.F, d.Fs);
    lo.R = T * d.k + (has_shared ? T : 0);
    const size_t nb = (size_t)perm_blocks(T);
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o += up(bytes);
        return at;
    };
    lo.x16 = take(d.f32 ? 0 : (size_t)T * d.H * 2);
    lo.z32 = take((size_t)T * d.Lz * 4);
    lo.z16 = take(d.f32 ? 0 : (size_t)T * d.Lz * 2);
    lo.z16h = take(lo.decode_path && d.mx ? (size_t)T * d.Lz * 2 : 0);  // fp16 z for 4-bit small batches
    lo.zlo = take(d.f32 || T <= kStreamMaxT ? 0 : (size_t)T * d.Lz * 2);  // low bf16 half of z (router input)
    lo.logits = take((size_t)T * d.E * 4 * (halves ? 2 : 1));  // folded router: hi and lo halves
    lo.ids = take((size_t)T * d.k * 4);
    lo.w = take((size_t)T * d.k * 4);
    lo.offsets = take((size_t)(d.E + 1) * 4);
    lo.perm = take((size_t)T * d.k * 4);
    lo.inv = take((size_t)T * d.k * 4);
    lo.rowinfo = take(lo.decode_path ? (size_t)T * d.k * 8 : 0);
    lo.hist = take(nb * d.E * 4);
    lo.base = take(nb * d.E * 4);
    lo.tiles = take((size_t)lo.max_tiles * sizeof(Tile));
    lo.ntiles = take(4);
    lo.H = take((size_t)lo.R * lo.Hs * act);
    lo.Y = take(lo.decode_path ? 0 : (size_t)lo.R * d.L * (d.f32 ? 4 : 2));
    lo.mpart = take(lo.decode_path ? (size_t)decode_groups() * T * d.Lz * 2 : 0);
    // merged rows (larger batches), or with expert groups and small batches whose U launch cannot
    // stage all groups at once, the U products of the groups [G][T][H] fp32
    lo.m = take(lo.decode_path ? (small_proj_fits(T, d.Lz) ? 0 : (size_t)d.G * T * d.H * 4) : (size_t)T * d.Lz * act);
    lo.deq = take(deq ? (size_t)d.E * 3 * d.F * d.L * 2 : 0);  // decoded bf16 records
    lo.deq_ts = take(deq ? (size_t)d.E * 3 * 4 : 0);
    lo.z8 = take(lo.mx_path ? (size_t)T * d.Lz : 0);
    lo.z8s = take(lo.mx_path ? (size_t)T * d.Lz / 32 : 0);
    lo.z4 = take(lo.mx_path ? (size_t)T * d.Lz / 2 : 0);
    lo.z4s = take(lo.mx_path ? (size_t)T * d.Lz / 32 : 0);
    lo.h8 = take(lo.mx_path ? (size_t)T * d.k * d.F : 0);
    lo.h8s = take(lo.mx_path ? (size_t)T * d.k * d.F / 32 : 0);
    lo.h4 = take(lo.mx_path ? (size_t)T * d.k * d.F / 2 : 0);
    lo.h4s = take(lo.mx_path ? (size_t)T * d.k * d.F / 32 : 0);
    lo.h16 = take(lo.mx_path ? (size_t)T * d.k * d.F * 2 : 0);
    lo.total = o;
    return lo;
}

size_t permute_ws(const Dims& d, int T) {
    const size_t nb = (size_t)perm_blocks(T);
    return nb <= 1 ? 0 : 2 * up(nb * d.E * 4);
}

size_t record_bytes(const Dims& d, bool shared) {
    const size_t F = shared ? d.Fs : d.F;
    if (shared || !d.mx) return 3 * F * d.L * (d.f32 ? 4 : 2);
    if (d.fmt == 2) return 3 * (F * d.L / 2) + 3 * (F * d.L / 16) + 16;  // + three fp32 tensor scales, padded
    return 3 * (F * d.L / 2) + 3 * (F * d.L / 32);
}

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    const char* pa = static_cast<const char*>(a);
    const char* pb = static_cast<const char*>(b);
    return pa < pb + nb && pb < pa + na;
}

// Workspace of lmoe_forward_noalloc: one array per GPU, allocated when the code object is loaded
// and held until the process ends.  Host code never passes its name to a kernel (that would be a
// host-side stand-in, not a device address): it uses the address hipGetSymbolAddress returns.
static __device__ __align__(256) unsigned char scratch[LMOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices] = {};
std::mutex g_scratch_mu;

// The device address of the current device's scratch array, looked up once per device (with
// that device current) and kept.
lmoe_status scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(LMOE_ERR_UNSUPPORTED, "device index %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!ptr) return fail(LMOE_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return LMOE_OK;
}

}  // namespace

extern "C" {

size_t lmoe_expert_record_bytes(const lmoe_config* cfg, int32_t shared) {
    Dims d;
    if (check_config(cfg, d) != LMOE_OK) return 0;
    if (shared && d.Fs == 0) return 0;
    return record_bytes(d, shared != 0);
}

lmoe_status lmoe_pack_experts(const lmoe_config* cfg, int32_t shared, const void* src, void* dst, int32_t n_records,
                              void* stream) {
    Dims d;
    lmoe_status st = check_config(cfg, d);
    if (st != LMOE_OK) return st;
    if (d.f32) return fail(LMOE_ERR_UNSUPPORTED, "fp32 records are read row-major and are not packed");
    if (shared && d.Fs == 0) return fail(LMOE_ERR_SHAPE, "shared_ffn is 0: there is no shared record");
    if (n_records < 0 || n_records > 65535 || (shared && n_records > 1))
        return fail(LMOE_ERR_SHAPE, "n_records must be in [0, 65535] (at most 1 shared record; got %d)", n_records);
    if (n_records == 0) return LMOE_OK;
    if (!src || !dst) return fail(LMOE_ERR_NULL, "src and dst must be non-NULL");
    if (!aligned16(src) || !aligned16(dst)) return fail(LMOE_ERR_ALIGN, "src and dst must be 16-byte aligned");
    const size_t rec = record_bytes(d, shared != 0);
    if (overlap(src, rec * n_records, dst, rec * n_records))
        return fail(LMOE_ERR_UNSUPPORTED, "src and dst overlap (packing is not in place)");
    const hipError_t e = launch_pack(src, dst, rec, n_records, shared ? d.Fs : d.F, d.L, shared ? 0 : d.fmt,
                                     static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "pack experts");
    return LMOE_OK;
}

size_t lmoe_fold_router_bytes(const lmoe_config* cfg) {
    Dims d;
    if (check_config(cfg, d) != LMOE_OK || d.f32) return 0;
    return (size_t)d.E * 2 * d.H * 2;
}

lmoe_status lmoe_fold_router(const lmoe_config* cfg, const void* D, const void* Wr, void* Gr, void* stream) {
    Dims d;
    lmoe_status st = check_config(cfg, d);
    if (st != LMOE_OK) return st;
    if (d.f32) return fail(LMOE_ERR_UNSUPPORTED, "the folded router is for bf16 dense weights");
    if (!D || !Wr || !Gr) return fail(LMOE_ERR_NULL, "D, Wr and Gr must be non-NULL");
    if (!aligned16(D) || !aligned16(Wr) || !aligned16(Gr)) return fail(LMOE_ERR_ALIGN, "D, Wr and Gr must be 16-byte aligned");
    const size_t gb = (size_t)d.E * 2 * d.H * 2;
    if (overlap(Gr, gb, D, (size_t)d.Lz * d.H * 2) || overlap(Gr, gb, Wr, (size_t)d.E * d.L * 2))
        return fail(LMOE_ERR_UNSUPPORTED, "Gr overlaps D or Wr");
    const hipError_t e = launch_fold_router(static_cast<const uint16_t*>(D), static_cast<const uint16_t*>(Wr), d.E, d.L,
                                            d.H, static_cast<uint16_t*>(Gr), static_cast<hipStream_t>(stream), d.Eg);
    if (e != hipSuccess) return hip_fail(e, "fold router");
    return LMOE_OK;
}

lmoe_status lmoe_workspace_bytes(const lmoe_config* cfg, int32_t T, size_t* bytes) {
    Dims d;
    lmoe_status st = check_config(cfg, d);
    if (st != LMOE_OK) return st;
    if ((st = check_T(d, T)) != LMOE_OK) return st;
    if (!bytes) return fail(LMOE_ERR_NULL, "bytes is NULL");
    // the small-batch partials can exceed what a slightly larger batch needs: report the maximum
    // over every T' <= T so that one workspace sized for a largest batch serves all smaller ones
    *bytes = std::max({plan(d, T).total, plan(d, std::min<int32_t>(T, kStreamMaxT)).total,
                       plan(d, std::min<int32_t>(T, kDecodeMaxT)).total});
    return LMOE_OK;
}

lmoe_status lmoe_permute_workspace_bytes(const lmoe_config* cfg, int32_t T, size_t* bytes) {
    Dims d;
    lmoe_status st = check_config(cfg, d);
    if (st != LMOE_OK) return st;
    if ((st = check_T(d, T)) != LMOE_OK) return st;
    if (!bytes) return fail(LMOE_ERR_NULL, "bytes is NULL");
    *bytes = permute_ws(d, T);
    return LMOE_OK;
}

lmoe_status lmoe_route(const lmoe_config* cfg, const lmoe_weights* weights, const float* z, int32_t T, int32_t* ids,
                       float* w, void* ws, size_t ws_bytes, void* stream) {
    Dims d;
    lmoe_status st = check_config(cfg, d);
    if (st != LMOE_OK) return st;
    if ((st = check_T(d, T)) != LMOE_OK) return st;
    if (!weights) return fail(LMOE_ERR_NULL, "weights is NULL");
    if (d.G > 1) return fail(LMOE_ERR_UNSUPPORTED, "lmoe_route takes one latent (one expert group)");
    if (T == 0) return LMOE_OK;
    if (!weights->Wr || !z || !ids || !w || !ws) return fail(LMOE_ERR_NULL, "Wr, z, ids, w and ws must be non-NULL");
    if (!aligned16(weights->Wr) || !aligned16(z) || !aligned16(ids) || !aligned16(w) || !aligned16(ws) ||
        (reinterpret_cast<uintptr_t>(weights->br) & 3u))
        return fail(LMOE_ERR_ALIGN, "tensor pointers must be 16-byte aligned (br 4-byte)");
    const size_t need = (size_t)T * d.E * 4;
    if (ws_bytes < need) return fail(LMOE_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
    hipStream_t s = static_cast<hipStream_t>(stream);
    float* logits = static_cast<float*>(ws);
    hipError_t e = d.f32 ? launch_proj_f32(z, static_cast<const float*>(weights->Wr), weights->br, T, d.E, d.L, 0, logits, s)
                         : launch_router_bf16(z, static_cast<const uint16_t*>(weights->Wr), weights->br, T, d.E, d.L,
                                              logits, s);
    if (e != hipSuccess) return hip_fail(e, "router logits");
    if ((e = launch_topk(logits, T, d.E, d.k, ids, w, s)) != hipSuccess) return hip_fail(e, "top-k");
    return LMOE_OK;
}

lmoe_status lmoe_permute(const lmoe_config* cfg, const int32_t* ids, int32_t T, int32_t* offsets, int32_t* perm,
                         int32_t* inv, void* ws, size_t ws_bytes, void* stream) {
    Dims d;
    lmoe_status st = check_config(cfg, d);
    if (st != LMOE_OK) return st;
    if ((st = check_T(d, T)) != LMOE_OK) return st;
    if (!offsets) return fail(LMOE_ERR_NULL, "offsets is NULL");
    if (T > 0 && (!ids || !perm || !inv)) return fail(LMOE_ERR_NULL, "ids, perm and inv must be non-NULL");
    if (!aligned16(ids) || !aligned16(offsets) || !aligned16(perm) || !aligned16(inv) || !aligned16(ws))
        return fail(LMOE_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
    const size_t need = permute_ws(d, T);
    if (need && (!ws || ws_bytes < need))
        return fail(LMOE_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws ? ws_bytes : 0, need);
    hipStream_t s = static_cast<hipStream_t>(stream);
    int32_t* hist = static_cast<int32_t*>(ws);
    int32_t* base = need ? reinterpret_cast<int32_t*>(static_cast<char*>(ws) + need / 2) : nullptr;
    const hipError_t e =
        launch_permute(ids, T, d.k, d.E, hist, base, offsets, perm, inv, 16, nullptr, nullptr, 0, s);
    if (e != hipSuccess) return hip_fail(e, "permute");
    return LMOE_OK;
}

}  // extern "C"

namespace {

// Every host-side check of lmoe_forward's arguments except the workspace's (shared with
// lmoe_forward_noalloc, which runs them before it looks up its device array).
lmoe_status check_forward(const lmoe_config* cfg, const lmoe_weights* wt, const void* x, int32_t T, const void* y,
                          const lmoe_forward_opts& o, Dims& d) {
    lmoe_status st = check_config(cfg, d);
    if (st != LMOE_OK) return st;
    if ((st = check_T(d, T)) != LMOE_OK) return st;
    if (!wt) return fail(LMOE_ERR_NULL, "weights is NULL");
    if (o.prenorm && d.f32) return fail(LMOE_ERR_UNSUPPORTED, "prenorm needs act BF16 (the block input is bf16(RMSNorm(h)))");
    if (T == 0) return LMOE_OK;
    if (!x || !y || !wt->D || !wt->U || !wt->Wr || !wt->experts)
        return fail(LMOE_ERR_NULL, "x, y, D, U, Wr and experts must be non-NULL");
    if (d.Fs > 0 && !wt->shared) return fail(LMOE_ERR_NULL, "shared_ffn > 0 but the shared expert record is NULL");
    if (d.G > 1 && !wt->Gr) return fail(LMOE_ERR_UNSUPPORTED, "expert groups need the folded router (weights->Gr)");
    const void* ptrs[] = {x, y, wt->D, wt->U, wt->Wr, wt->Gr, wt->experts, wt->shared, o.aux_z, o.aux_ids, o.aux_w,
                          o.aux_offsets, o.aux_perm};
    for (const void* p : ptrs)
        if (!aligned16(p)) return fail(LMOE_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
    if (reinterpret_cast<uintptr_t>(wt->br) & 3u) return fail(LMOE_ERR_ALIGN, "br must be 4-byte aligned");
    const size_t xbytes = (size_t)T * d.H * ((o.prenorm || d.f32) ? 4 : 2);
    const size_t ybytes = (size_t)T * d.H * ((o.residual || d.f32) ? 4 : 2);
    if (overlap(x, xbytes, y, ybytes) && !(x == y && o.prenorm && o.residual))
        return fail(LMOE_ERR_UNSUPPORTED, "x and y overlap (only x == y with prenorm and residual is allowed)");
    return LMOE_OK;
}

}  // namespace

extern "C" {

lmoe_status lmoe_forward(const lmoe_config* cfg, const lmoe_weights* wt, const void* x, int32_t T, void* y,
                         const lmoe_forward_opts* opts, void* ws, size_t ws_bytes, void* stream) {
    Dims d;
    const lmoe_forward_opts none{};
    const lmoe_forward_opts& o = opts ? *opts : none;
    lmoe_status st = check_forward(cfg, wt, x, T, y, o, d);
    if (st != LMOE_OK || T == 0) return st;
    if (!aligned16(ws)) return fail(LMOE_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
    const Layout lo = plan(d, T);
    if (!ws || ws_bytes < lo.total)
        return fail(LMOE_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws ? ws_bytes : 0, lo.total);

    hipStream_t s = static_cast<hipStream_t>(stream);
    StageEvents ev(o.stage_events, s);
    char* W = static_cast<char*>(ws);
    auto at = [&](size_t off) { return static_cast<void*>(W + off); };
    float* z32 = o.aux_z ? o.aux_z : static_cast<float*>(at(lo.z32));
    float* logits = static_cast<float*>(at(lo.logits));
    int32_t* ids = o.aux_ids ? o.aux_ids : static_cast<int32_t*>(at(lo.ids));
    float* wts = o.aux_w ? o.aux_w : static_cast<float*>(at(lo.w));
    int32_t* offsets = o.aux_offsets ? o.aux_offsets : static_cast<int32_t*>(at(lo.offsets));
    int32_t* perm = o.aux_perm ? o.aux_perm : static_cast<int32_t*>(at(lo.perm));
    int32_t* inv = static_cast<int32_t*>(at(lo.inv));
    int32_t* hist = static_cast<int32_t*>(at(lo.hist));
    int32_t* base = static_cast<int32_t*>(at(lo.base));
    Tile* tiles = static_cast<Tile*>(at(lo.tiles));
    int32_t* ntiles = static_cast<int32_t*>(at(lo.ntiles));
    void* Y = at(lo.Y);  // fp32 rows on the fp32 path, bf16 rows otherwise
    const int has_shared = d.Fs > 0;
    hipError_t e;

    if (d.f32) {
        const float* xf = static_cast<const float*>(x);
        ev.begin(LMOE_STAGE_D);
        if ((e = launch_proj_f32(xf, static_cast<const float*>(wt->D), nullptr, T, d.L, d.H, 0, z32, s)) != hipSuccess)
            return hip_fail(e, "D projection");
        ev.end(LMOE_STAGE_D);
        ev.begin(LMOE_STAGE_ROUTER);
        if ((e = launch_proj_f32(z32, static_cast<const float*>(wt->Wr), wt->br, T, d.E, d.L, 0, logits, s)) != hipSuccess)
            return hip_fail(e, "router logits");
        ev.end(LMOE_STAGE_ROUTER);
        ev.begin(LMOE_STAGE_TOPK);
        if ((e = launch_topk(logits, T, d.E, d.k, ids, wts, s)) != hipSuccess) return hip_fail(e, "top-k");
        ev.end(LMOE_STAGE_TOPK);
        ev.begin(LMOE_STAGE_PERMUTE);
        if ((e = launch_permute(ids, T, d.k, d.E, hist, base, offsets, perm, inv, lo.BM, nullptr, nullptr, has_shared,
                                s)) != hipSuccess)
            return hip_fail(e, "permute");
        ev.end(LMOE_STAGE_PERMUTE);
        F32ExpertArgs a{z32, ids, perm, static_cast<const float*>(wt->experts), static_cast<const float*>(wt->shared),
                        T, d.k, d.L, d.F, d.Fs, lo.Hs, static_cast<float*>(at(lo.H)), static_cast<float*>(Y)};
        if ((e = launch_experts_f32(a, s, ev)) != hipSuccess) return hip_fail(e, "experts");
        float* m = static_cast<float*>(at(lo.m));
        ev.begin(LMOE_STAGE_COMBINE);
        if ((e = launch_combine(Y, wts, T, d.k, d.L, has_shared, false, m, s)) != hipSuccess) return hip_fail(e, "combine");
        ev.end(LMOE_STAGE_COMBINE);
        ev.begin(LMOE_STAGE_U);
        if ((e = launch_proj_f32(m, static_cast<const float*>(wt->U), nullptr, T, d.H, d.L, o.residual ? 2 : 0,
                                 static_cast<float*>(y), s)) != hipSuccess)
            return hip_fail(e, "U projection");
        ev.end(LMOE_STAGE_U);
        return ev.err != hipSuccess ? hip_fail(ev.err, "stage event record") : LMOE_OK;
    }

    const uint16_t* x16 = static_cast<const uint16_t*>(x);
    // small batches whose D launch stages its input in LDS form bf16(RMSNorm(h)) there
    const bool fused_d_router = wt->Gr && lo.fused_router;
    const bool norm_in_d = o.prenorm && (fused_d_router || (T <= kStreamMaxT && small_proj_fits(T, d.H)));
    const float* hnorm = norm_in_d ? static_cast<const float*>(x) : nullptr;
    if (o.prenorm && !norm_in_d) {
        uint16_t* xn = static_cast<uint16_t*>(at(lo.x16));
        ev.begin(LMOE_STAGE_PRENORM);
        if ((e = launch_rmsnorm(static_cast<const float*>(x), T, d.H, xn, s)) != hipSuccess) return hip_fail(e, "rmsnorm");
        ev.end(LMOE_STAGE_PRENORM);
        x16 = xn;
    }
    uint16_t* z16 = static_cast<uint16_t*>(at(lo.z16));
    // fp16 z for the 4-bit experts of a small batch, written by the small-batch D launches
    uint16_t* z16h = lo.decode_path && d.mx ? static_cast<uint16_t*>(at(lo.z16h)) : nullptr;
    if (fused_d_router) {  // z and the logits (folded router) in one launch
        ev.begin(LMOE_STAGE_D);
        if ((e = launch_proj_router_bf16(x16, static_cast<const uint16_t*>(wt->D), static_cast<const uint16_t*>(wt->Gr),
                                         wt->br, T, d.Lz, d.H, d.E, z32, z16, logits, s, z16h, hnorm)) != hipSuccess)
            return hip_fail(e, "D projection and router logits");
        ev.end(LMOE_STAGE_D);
    } else {
        ev.begin(LMOE_STAGE_D);
        uint16_t* zlo = T > kStreamMaxT ? static_cast<uint16_t*>(at(lo.zlo)) : nullptr;
        if (!(T <= kStreamMaxT && small_proj_fits(T, d.H))) z16h = nullptr;  // only the small-batch D launch writes it
        // with the router reading the bf16 halves (zlo) and the experts z16, fp32 z is only
        // written when the caller asks for it
        float* zf = zlo && !o.aux_z ? nullptr : z32;
        if ((e = launch_proj_bf16(x16, static_cast<const uint16_t*>(wt->D), T, d.Lz, d.H, 0, zf, z16, s, zlo, z16h,
                                  hnorm)) != hipSuccess)
            return hip_fail(e, "D projection");
        ev.end(LMOE_STAGE_D);
        ev.begin(LMOE_STAGE_ROUTER);
        if (d.G > 1)  // each expert reads its own group's latent: the logits come from x and Gr
            e = launch_router_x(x16, static_cast<const uint16_t*>(wt->Gr), wt->br, T, d.E, d.H, logits, s);
        else
            e = launch_router_bf16(z32, static_cast<const uint16_t*>(wt->Wr), wt->br, T, d.E, d.L, logits, s,
                                   zlo ? z16 : nullptr, zlo);
        if (e != hipSuccess) return hip_fail(e, "router logits");
        ev.end(LMOE_STAGE_ROUTER);
    }
    // top-k and permutation: for small batches inside the gate/up launch, else one launch for
    // T <= 64 (the TOPK stage events bracket both) or several
    const float* logits2 = fused_d_router || d.G > 1 || T > kStreamMaxT ? logits + (size_t)T * d.E : nullptr;
    int2* rowinfo = lo.decode_path ? static_cast<int2*>(at(lo.rowinfo)) : nullptr;
    const ExpertRoute route{logits, logits2, lo.BM, has_shared, RouteOut{ids, wts, offsets, perm, inv, tiles, ntiles, rowinfo}};
    const bool route_in_experts = lo.decode_path && kRouteInExperts;
    if (!route_in_experts) {
        ev.begin(LMOE_STAGE_TOPK);
        if ((e = launch_topk_permute(logits, T, d.E, d.k, ids, wts, hist, base, offsets, perm, inv, lo.BM, tiles, ntiles,
                                     has_shared, s, logits2, rowinfo)) != hipSuccess)
            return hip_fail(e, "top-k / permute");
        ev.end(LMOE_STAGE_TOPK);
    }
    uint16_t* mpart = static_cast<uint16_t*>(at(lo.mpart));
    ExpertArgs a{tiles, ntiles, perm, T, d.k, d.E, d.L, d.F, d.Fs, lo.Hs, z16, z16h, wt->experts, record_bytes(d, false),
                 wt->shared, static_cast<uint16_t*>(at(lo.H)), static_cast<uint16_t*>(Y), lo.max_tiles, lo.stream_path,
                 lo.decode_path, d.fmt, mpart, wts, rowinfo, route_in_experts ? &route : nullptr, d.Eg, d.Lz,
                 lo.deq_path ? static_cast<uint16_t*>(at(lo.deq)) : nullptr,
                 lo.deq_path ? static_cast<float*>(at(lo.deq_ts)) : nullptr, offsets};
    a.tile_rows = lo.BM;
    if (lo.mx_path) {
        a.mx_path = true;
        a.z8 = static_cast<uint8_t*>(at(lo.z8));
        a.z8s = static_cast<uint8_t*>(at(lo.z8s));
        a.z4 = static_cast<uint8_t*>(at(lo.z4));
        a.z4s = static_cast<uint8_t*>(at(lo.z4s));
        a.h8 = static_cast<uint8_t*>(at(lo.h8));
        a.h8s = static_cast<uint8_t*>(at(lo.h8s));
        a.h4 = static_cast<uint8_t*>(at(lo.h4));
        a.h4s = static_cast<uint8_t*>(at(lo.h4s));
        a.h16 = static_cast<uint16_t*>(at(lo.h16));
    }
    if ((e = launch_experts_bf16(a, s, ev)) != hipSuccess) return hip_fail(e, "experts");
    const int umode = o.residual ? 2 : 1;
    const uint16_t* U = static_cast<const uint16_t*>(wt->U);
    if (lo.decode_path) {  // the down launch merged the rows into partials; U sums them
        ev.begin(LMOE_STAGE_U);
        if (small_proj_fits(T, d.Lz)) {
            e = launch_proj_partials(mpart, decode_groups(), U, T, d.H, d.Lz, umode, static_cast<float*>(y),
                                     static_cast<uint16_t*>(y), s);
        } else {  // expert groups: U_g . m_g per group (K = latent each), then the sum over groups
            e = launch_proj_partials_kgroups(mpart, decode_groups(), U, T, d.H, d.L, d.G, static_cast<float*>(at(lo.m)),
                                             umode, static_cast<float*>(y), static_cast<uint16_t*>(y), s);
        }
        if (e != hipSuccess) return hip_fail(e, "U projection");
        ev.end(LMOE_STAGE_U);
        return ev.err != hipSuccess ? hip_fail(ev.err, "stage event record") : LMOE_OK;
    }
    uint16_t* m16 = static_cast<uint16_t*>(at(lo.m));
    ev.begin(LMOE_STAGE_COMBINE);
    if ((e = launch_combine(Y, wts, T, d.k, d.L, has_shared, true, m16, s, ids, d.G, d.Eg)) != hipSuccess)
        return hip_fail(e, "combine");
    ev.end(LMOE_STAGE_COMBINE);
    ev.begin(LMOE_STAGE_U);
    if ((e = launch_proj_bf16(m16, U, T, d.H, d.Lz, umode, static_cast<float*>(y), static_cast<uint16_t*>(y), s)) !=
        hipSuccess)
        return hip_fail(e, "U projection");
    ev.end(LMOE_STAGE_U);
    return ev.err != hipSuccess ? hip_fail(ev.err, "stage event record") : LMOE_OK;
}

lmoe_status lmoe_forward_noalloc(const lmoe_config* cfg, const lmoe_weights* weights, const void* x, int32_t T, void* y,
                                 const lmoe_forward_opts* opts, void* stream) {
    Dims d;
    const lmoe_forward_opts none{};
    lmoe_status st = check_forward(cfg, weights, x, T, y, opts ? *opts : none, d);
    if (st != LMOE_OK || T == 0) return st;
    const size_t need = plan(d, T).total;
    if (need > (size_t)LMOE_NOALLOC_SCRATCH_BYTES)
        return fail(LMOE_ERR_WORKSPACE,
                    "T = %d needs %zu workspace bytes, more than the %zu bytes of the allocation-free entry point",
                    T, need, (size_t)LMOE_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    if ((st = scratch_address(&ws)) != LMOE_OK) return st;
    return lmoe_forward(cfg, weights, x, T, y, opts, ws, (size_t)LMOE_NOALLOC_SCRATCH_BYTES, stream);
}

const char* lmoe_status_str(lmoe_status status) {
    // read as an integer: a C caller may pass any int, which C++ does not allow an enum to hold
    int32_t v;
    memcpy(&v, &status, sizeof v);
    switch (v) {
        case LMOE_OK: return "ok";
        case LMOE_ERR_NULL: return "required pointer is NULL";
        case LMOE_ERR_SHAPE: return "dimension out of range or inconsistent";
        case LMOE_ERR_DTYPE: return "unknown dtype";
        case LMOE_ERR_ALIGN: return "pointer not 16-byte aligned";
        case LMOE_ERR_WORKSPACE: return "workspace missing or too small";
        case LMOE_ERR_UNSUPPORTED: return "unsupported combination";
        case LMOE_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char* lmoe_last_error(void) { return g_err.c_str(); }

int32_t lmoe_version(void) { return 100; }

}  // extern "C"
