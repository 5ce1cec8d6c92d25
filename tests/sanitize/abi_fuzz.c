/* Host-side fuzz of the C ABI in include/lmoe.h, built with AddressSanitizer and
 * UndefinedBehaviorSanitizer on the host code (see tests/test_abi_sanitize.py).
 *
 * Only host logic is exercised: the size queries over a seeded grid of configurations (valid,
 * inconsistent and extreme values), and every entry point with arguments that the host-side
 * validation must reject before anything is enqueued (NULL pointers, misaligned pointers, bad
 * dtypes, out-of-range sizes, short workspaces).  Buffers handed to the library are small heap
 * blocks, so any host read through them past their end is reported by the sanitizer.  The run
 * refuses to start when a GPU is visible, since no call here is meant to reach a device.
 *
 * Exit status: 0 = all checks passed, 1 = a check failed, 77 = skipped (GPU visible).
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "lmoe.h"

extern int hipGetDeviceCount(int* count);

static int failures = 0;
#define CHECK(cond, ...)                               \
    do {                                               \
        if (!(cond)) {                                 \
            fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
            fprintf(stderr, __VA_ARGS__);              \
            fprintf(stderr, "\n");                     \
            ++failures;                                \
        }                                              \
    } while (0)

static uint64_t rng_state = 0x4C4D4F45u;
static uint32_t rnd(void) { /* xorshift64* */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (uint32_t)((rng_state * 2685821657736338717ull) >> 32);
}
static int32_t pick(const int32_t* v, int n) { return v[rnd() % (uint32_t)n]; }

static const int32_t kDims[] = {-7, -1, 0, 1, 2, 16, 63, 64, 100, 128, 192, 256, 640, 1280, 1792, 2560,
                                4096, 14336, 1 << 20, 1 << 30, INT32_MAX, INT32_MIN};
static const int32_t kSmall[] = {-1, 0, 1, 2, 3, 8, 10, 16, 17, 64, 512, 1024, 1025, INT32_MAX};
static const int32_t kDtypes[] = {-1, LMOE_F32, LMOE_BF16, LMOE_MXFP4, LMOE_NVFP4, 4, 99};
static const int32_t kT[] = {-1, 0, 1, 8, 16, 17, 64, 65, 95, 96, 383, 384, 4096, 16384, 1 << 20, (1 << 20) + 1,
                             INT32_MAX, INT32_MIN};

static lmoe_config valid_cfg(void) {
    lmoe_config c;
    memset(&c, 0, sizeof c);
    c.hidden = 2560;
    c.latent = 1792;
    c.n_experts = 512;
    c.top_k = 10;
    c.ffn = 640;
    c.shared_ffn = 640;
    c.act_dtype = LMOE_BF16;
    c.dense_dtype = LMOE_BF16;
    c.expert_dtype = LMOE_BF16;
    c.groups = 1;
    c.mx_mfma_min_t = 0;
    return c;
}

static lmoe_config random_cfg(void) {
    lmoe_config c = valid_cfg();
    /* perturb a random subset of the fields */
    const uint32_t mask = rnd();
    if (mask & 1) c.hidden = pick(kDims, sizeof kDims / 4);
    if (mask & 2) c.latent = pick(kDims, sizeof kDims / 4);
    if (mask & 4) c.n_experts = pick(kSmall, sizeof kSmall / 4);
    if (mask & 8) c.top_k = pick(kSmall, sizeof kSmall / 4);
    if (mask & 16) c.ffn = pick(kDims, sizeof kDims / 4);
    if (mask & 32) c.shared_ffn = pick(kDims, sizeof kDims / 4);
    if (mask & 64) c.act_dtype = pick(kDtypes, sizeof kDtypes / 4);
    if (mask & 128) c.dense_dtype = pick(kDtypes, sizeof kDtypes / 4);
    if (mask & 256) c.expert_dtype = pick(kDtypes, sizeof kDtypes / 4);
    if (mask & 512) c.groups = pick(kSmall, sizeof kSmall / 4);
    if (mask & 1024) c.mx_mfma_min_t = pick(kT, sizeof kT / 4);
    return c;
}

static void size_queries(void) {
    size_t n = 0;
    CHECK(lmoe_workspace_bytes(NULL, 8, &n) == LMOE_ERR_NULL, "NULL cfg");
    lmoe_config c = valid_cfg();
    CHECK(lmoe_workspace_bytes(&c, 8, NULL) == LMOE_ERR_NULL, "NULL bytes");
    CHECK(lmoe_permute_workspace_bytes(&c, 8, NULL) == LMOE_ERR_NULL, "NULL bytes");
    CHECK(lmoe_expert_record_bytes(NULL, 0) == 0, "NULL cfg record bytes");
    CHECK(lmoe_fold_router_bytes(NULL) == 0, "NULL cfg fold bytes");
    long ok = 0;
    for (int it = 0; it < 200000; ++it) {
        lmoe_config r = random_cfg();
        const int32_t T = pick(kT, sizeof kT / 4);
        size_t a = 0, b = 0;
        const lmoe_status s1 = lmoe_workspace_bytes(&r, T, &a);
        const lmoe_status s2 = lmoe_permute_workspace_bytes(&r, T, &b);
        CHECK(s1 >= LMOE_OK && s1 <= LMOE_ERR_HIP, "status %d", (int)s1);
        CHECK(s2 >= LMOE_OK && s2 <= LMOE_ERR_HIP, "status %d", (int)s2);
        if (s1 == LMOE_OK) {
            ++ok;
            CHECK(T >= 0 && T <= (1 << 20), "workspace accepted T=%d", T);
            CHECK(a % 256 == 0, "workspace size %zu not a multiple of 256", a);
        } else {
            CHECK(strlen(lmoe_last_error()) > 0, "no message for status %d", (int)s1);
        }
        (void)lmoe_expert_record_bytes(&r, 0);
        (void)lmoe_expert_record_bytes(&r, 1);
        (void)lmoe_fold_router_bytes(&r);
    }
    CHECK(ok > 1000, "only %ld configurations accepted", ok);
    printf("size queries: 200000 random configurations, %ld accepted\n", ok);
}

/* Every entry point with arguments that validation rejects.  `blk` is a 64-byte heap block used as
 * every device pointer but x and y, `blk + 1` as a misaligned one; x and y sit 32 MB apart in one
 * larger block (so that their T x hidden ranges do not overlap).  Nothing may be read through
 * any of them. */
static void rejected_calls(void) {
    unsigned char* blk = (unsigned char*)malloc(64);
    unsigned char* io = (unsigned char*)malloc((size_t)64 << 20);
    void* p = blk;
    void* mis = blk + 1;
    void* x = io;
    void* y = io + ((size_t)32 << 20);
    lmoe_config c = valid_cfg();
    lmoe_weights w;
    memset(&w, 0, sizeof w);
    w.D = p;
    w.U = p;
    w.Wr = p;
    w.br = (const float*)p;
    w.shared = p;
    w.experts = p;
    w.Gr = p;
    lmoe_forward_opts o;
    memset(&o, 0, sizeof o);
    const int32_t T = 8;
    size_t need = 0;
    CHECK(lmoe_workspace_bytes(&c, T, &need) == LMOE_OK && need > 64, "workspace query");

    /* NULL arguments */
    CHECK(lmoe_forward(NULL, &w, x, T, y, &o, p, need, NULL) == LMOE_ERR_NULL, "forward NULL cfg");
    CHECK(lmoe_forward(&c, NULL, x, T, y, &o, p, need, NULL) == LMOE_ERR_NULL, "forward NULL weights");
    CHECK(lmoe_forward(&c, &w, NULL, T, y, &o, p, need, NULL) == LMOE_ERR_NULL, "forward NULL x");
    CHECK(lmoe_forward(&c, &w, x, T, NULL, &o, p, need, NULL) == LMOE_ERR_NULL, "forward NULL y");
    CHECK(lmoe_forward_noalloc(NULL, &w, x, T, y, &o, NULL) == LMOE_ERR_NULL, "noalloc NULL cfg");
    CHECK(lmoe_forward_noalloc(&c, &w, NULL, T, y, &o, NULL) == LMOE_ERR_NULL, "noalloc NULL x");
    CHECK(lmoe_route(NULL, &w, (const float*)p, T, (int32_t*)p, (float*)p, p, need, NULL) == LMOE_ERR_NULL, "route");
    CHECK(lmoe_route(&c, &w, NULL, T, (int32_t*)p, (float*)p, p, need, NULL) == LMOE_ERR_NULL, "route NULL z");
    CHECK(lmoe_permute(NULL, (const int32_t*)p, T, (int32_t*)p, (int32_t*)p, (int32_t*)p, NULL, 0, NULL) ==
              LMOE_ERR_NULL, "permute NULL cfg");
    CHECK(lmoe_permute(&c, NULL, T, (int32_t*)p, (int32_t*)p, (int32_t*)p, NULL, 0, NULL) == LMOE_ERR_NULL,
          "permute NULL ids");
    CHECK(lmoe_pack_experts(NULL, 0, p, p, 1, NULL) == LMOE_ERR_NULL, "pack NULL cfg");
    CHECK(lmoe_pack_experts(&c, 0, NULL, p, 1, NULL) == LMOE_ERR_NULL, "pack NULL src");
    CHECK(lmoe_fold_router(NULL, p, p, p, NULL) == LMOE_ERR_NULL, "fold NULL cfg");
    CHECK(lmoe_fold_router(&c, p, NULL, p, NULL) == LMOE_ERR_NULL, "fold NULL Wr");

    /* misaligned pointers */
    CHECK(lmoe_forward(&c, &w, (unsigned char*)x + 1, T, y, &o, p, need, NULL) == LMOE_ERR_ALIGN, "forward misaligned x");
    CHECK(lmoe_forward(&c, &w, x, T, (unsigned char*)y + 1, &o, p, need, NULL) == LMOE_ERR_ALIGN, "forward misaligned y");
    CHECK(lmoe_forward(&c, &w, x, T, y, &o, mis, need, NULL) == LMOE_ERR_ALIGN, "forward misaligned ws");
    lmoe_weights wm = w;
    wm.experts = mis;
    CHECK(lmoe_forward(&c, &wm, x, T, y, &o, p, need, NULL) == LMOE_ERR_ALIGN, "forward misaligned experts");
    CHECK(lmoe_pack_experts(&c, 0, mis, p, 1, NULL) == LMOE_ERR_ALIGN, "pack misaligned src");

    /* sizes */
    CHECK(lmoe_forward(&c, &w, x, -1, y, &o, p, need, NULL) == LMOE_ERR_SHAPE, "forward T=-1");
    CHECK(lmoe_forward(&c, &w, x, (1 << 20) + 1, y, &o, p, need, NULL) == LMOE_ERR_SHAPE, "forward T too large");
    CHECK(lmoe_forward(&c, &w, x, T, y, &o, p, need - 1, NULL) == LMOE_ERR_WORKSPACE, "forward short ws");
    CHECK(lmoe_forward(&c, &w, x, T, y, &o, NULL, need, NULL) != LMOE_OK, "forward NULL ws");
    CHECK(lmoe_forward_noalloc(&c, &w, x, 4096, y, &o, NULL) == LMOE_ERR_WORKSPACE, "noalloc beyond its array");
    CHECK(lmoe_pack_experts(&c, 0, p, p, -1, NULL) == LMOE_ERR_SHAPE, "pack n_records=-1");
    lmoe_config bad = c;
    bad.top_k = 0;
    CHECK(lmoe_forward(&bad, &w, x, T, y, &o, p, need, NULL) == LMOE_ERR_SHAPE, "k=0");
    bad = c;
    bad.top_k = bad.n_experts + 1;
    CHECK(lmoe_forward(&bad, &w, x, T, y, &o, p, need, NULL) == LMOE_ERR_SHAPE, "k>E");
    bad = c;
    bad.latent = 100;
    CHECK(lmoe_forward(&bad, &w, x, T, y, &o, p, need, NULL) == LMOE_ERR_SHAPE, "latent not a multiple of 64");
    bad = c;
    bad.expert_dtype = 9;
    CHECK(lmoe_forward(&bad, &w, x, T, y, &o, p, need, NULL) == LMOE_ERR_DTYPE, "unknown dtype");
    bad = c;
    bad.mx_mfma_min_t = -2;
    CHECK(lmoe_forward(&bad, &w, x, T, y, &o, p, need, NULL) == LMOE_ERR_SHAPE, "mx_mfma_min_t=-2");
    lmoe_weights ws_noshared = w;
    ws_noshared.shared = NULL;
    CHECK(lmoe_forward(&c, &ws_noshared, x, T, y, &o, p, need, NULL) == LMOE_ERR_NULL, "shared record missing");

    /* random invalid configurations on every entry point: whatever validation answers, it must
     * not be OK for a configuration the size query rejects */
    int rejected = 0;
    for (int it = 0; it < 20000; ++it) {
        lmoe_config r = random_cfg();
        const int32_t t = pick(kT, sizeof kT / 4);
        size_t nb = 0;
        if (lmoe_workspace_bytes(&r, t, &nb) == LMOE_OK) continue;
        ++rejected;
        CHECK(lmoe_forward(&r, &w, x, t, y, &o, p, (size_t)1 << 40, NULL) != LMOE_OK, "forward accepted");
        CHECK(lmoe_forward_noalloc(&r, &w, x, t, y, &o, NULL) != LMOE_OK, "noalloc accepted");
    }
    printf("rejected calls: fixed cases and %d random rejected configurations\n", rejected);

    for (int s = -3; s < 12; ++s) CHECK(lmoe_status_str((lmoe_status)s) != NULL, "status string %d", s);
    CHECK(lmoe_version() >= 100, "version");
    free(io);
    free(blk);
}

int main(void) {
    int n = 0;
    if (hipGetDeviceCount(&n) == 0 && n > 0) {
        printf("a GPU is visible: skipped (these calls are meant for a host without one)\n");
        return 77;
    }
    size_queries();
    rejected_calls();
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("all checks passed\n");
    return 0;
}
