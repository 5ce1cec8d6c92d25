/*
 * lmoe.h — C ABI of the latent-MoE feed-forward block for AMD Instinct MI355X (gfx950).
 *
 * The block is the one the Edge0-145B model-detail page describes in section "模型架构"
 * (Fig. 3 caption and the paragraph after it): a per-layer matrix D projects each token's
 * hidden state (2560-d) to the latent width l (1792); a router picks top_k (10) of
 * n_experts (512) experts; each picked expert is a SwiGLU l -> ffn (640) -> l; one shared
 * expert runs alongside; the merged result is projected back to the hidden width by the
 * per-layer matrix U.  Only the experts live in latent space; D and U are shared by all of
 * a layer's experts.
 *
 * Readings where the page is silent (stated once here, used by every call):
 *   - router logits = z . Wr^T + br (br optional), computed from the fp32 latent z;
 *   - top_k selection: largest logits, a lower expert id wins an exact tie; the ids of a
 *     token are returned in ascending expert id;
 *   - routing weights = softmax over the top_k selected logits (equivalently a softmax over
 *     all experts renormalised over the selected ones), so they sum to 1;
 *   - SwiGLU(z) = (SiLU(z gate^T) * (z up^T)) down^T, SiLU(v) = v / (1 + exp(-v)), no biases;
 *   - shared expert: weight 1, added to the routed sum before U;
 *   - merged m_t = shared_t + sum over slots (ascending expert id) of w_{t,s} * expert_s(z_t).
 *
 * Expert groups (lmoe_config.groups = G > 1): the sharing as the release report "1450 亿参数
 * 端侧模型 Edge0-145B 开源" describes it (section "Edge0 的内部机制": every 64 experts form a group
 * sharing one pair of large matrices).  Experts g*E/G .. (g+1)*E/G - 1 form group g, which owns
 * D_g and U_g; z_g = x D_g^T; expert e's router row and SwiGLU read its group's z_g, its
 * weighted output joins that group's merged row m_g, and y = sum_g m_g U_g^T.  The shared
 * expert counts as a member of group 0 (a reading: the pages do not place it).  G = 0 or 1 is
 * the single pair above.
 *
 * Conventions for every call
 *   - Every tensor argument is a caller-owned DEVICE pointer, row-major with the innermost
 *     dimension contiguous, 16-byte aligned.  Every weight matrix is stored output-major
 *     with its reduction dimension contiguous:
 *         D  [latent][hidden]     U  [hidden][latent]     Wr [n_experts][latent]
 *     With G expert groups, D is [G*latent][hidden] (group g's rows g*latent ..) and U is
 *     [hidden][G*latent] (group g's columns g*latent ..).
 *   - An expert record (routed experts and the shared expert) is contiguous:
 *         F32/BF16: gate [ffn][latent], up [ffn][latent], down [latent][ffn] elements;
 *         MXFP4 (routed experts only): gate nibbles [ffn][latent/2], up nibbles
 *             [ffn][latent/2], down nibbles [latent][ffn/2], then gate scales
 *             [ffn][latent/32], up scales [ffn][latent/32], down scales [latent][ffn/32].
 *             Elements are OCP MX FP4 E2M1 (low nibble = even K index), one E8M0 scale
 *             byte (value 2^(byte-127)) per 32 consecutive K values.
 *         NVFP4 (routed experts only): the three nibble arrays as for MXFP4, then gate scales
 *             [ffn][latent/16], up scales [ffn][latent/16], down scales [latent][ffn/16], one
 *             FP8 E4M3 byte per 16 consecutive K values, then the three matrices' fp32
 *             tensor scales (gate, up, down) and 4 zero bytes; element value =
 *             E2M1 * E4M3(block scale) * tensor scale.
 *     Routed experts are n_experts records back to back.  The shared expert record uses
 *     the dense dtype and shared_ffn in place of ffn.
 *   - lmoe_forward reads BF16 and MXFP4 records in the PACKED layout that lmoe_pack_experts
 *     writes (same size; F32 records stay row-major).  Packing permutes each matrix into
 *     1 KB tiles of 16 rows: BF16 tiles hold 16 rows x 32 columns, the 16-byte unit of row j
 *     and columns 8q..8q+7 at position 16q + j, tiles ordered by (row block, column step);
 *     4-bit nibble tiles hold 16 rows x 128 values (unit of row j, values 32q..32q+31 at
 *     position 16q + j) and each has a scale tile in the same unit order: MXFP4 one byte per
 *     unit (64 bytes), NVFP4 the unit's two E4M3 bytes (128 bytes); NVFP4 tensor scales stay
 *     at the end of the record.  A tile is the
 *     register image of one matrix-core operand, so the kernels read it with contiguous 1 KB
 *     wave loads.
 *   - BF16 tensors hold raw bf16 bit patterns (uint16).
 *   - All calls are asynchronous on `stream` (a hipStream_t passed as void*; NULL = the
 *     null stream), allocate nothing, never synchronise, keep no per-call state, and may be
 *     captured into a HIP graph.  Calls that share a workspace must be ordered.
 *   - Arguments are validated on the host before anything is enqueued.  On an error
 *     nothing is enqueued and no output is touched; lmoe_last_error() describes it.
 *     Launch failures reported by the HIP runtime map to LMOE_ERR_HIP.  Faults that
 *     happen while kernels run surface at the caller's next synchronisation.
 *   - NaN/Inf inputs are not checked; outputs are then undefined, but every kernel stays
 *     within the bounds of the buffers described here.  Batches of up to 64 tokens with 4-bit
 *     routed experts carry z and the SwiGLU rows in fp16 (11 significant bits) for those
 *     experts: magnitudes above 65504 saturate there (they stay finite but lose their size).
 *   - For identical inputs, configuration, T and device, outputs are bitwise identical
 *     (no floating-point atomics, fixed reduction orders).
 *
 * Supported dtype combinations (others return LMOE_ERR_UNSUPPORTED):
 *   act F32,  dense F32,  expert F32     (plain fp32 path)
 *   act BF16, dense BF16, expert BF16    (bf16 storage, fp32 accumulation)
 *   act BF16, dense BF16, expert MXFP4
 *   act BF16, dense BF16, expert NVFP4
 * Dimension limits: hidden, latent, ffn, shared_ffn multiples of 64 (shared_ffn may be 0;
 * with 4-bit experts latent, ffn and shared_ffn must be multiples of 128);
 * 1 <= top_k <= 16; top_k <= n_experts <= 1024; 0 <= T <= 2^20 with T*top_k < 2^31.
 * Expert groups: 1 <= groups <= 64 dividing n_experts; groups > 1 needs act and dense BF16
 * and a folded router (weights.Gr; otherwise LMOE_ERR_UNSUPPORTED), and lmoe_route, which
 * takes an fp32 latent, supports one group only.
 */
#ifndef LMOE_H
#define LMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    LMOE_OK = 0,
    LMOE_ERR_NULL = 1,        /* a required pointer is NULL */
    LMOE_ERR_SHAPE = 2,       /* a dimension is out of range or inconsistent */
    LMOE_ERR_DTYPE = 3,       /* an unknown dtype code */
    LMOE_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned */
    LMOE_ERR_WORKSPACE = 5,   /* workspace missing or smaller than the size query returns */
    LMOE_ERR_UNSUPPORTED = 6, /* valid but unsupported combination (dtypes, options) */
    LMOE_ERR_HIP = 7          /* the HIP runtime reported an error while enqueuing */
} lmoe_status;

typedef enum { LMOE_F32 = 0, LMOE_BF16 = 1, LMOE_MXFP4 = 2, LMOE_NVFP4 = 3 } lmoe_dtype;

typedef struct {
    int32_t hidden;       /* H: token width outside the expert pool (2560) */
    int32_t latent;       /* l: latent width (1792) */
    int32_t n_experts;    /* E: routed experts per layer (512) */
    int32_t top_k;        /* k: routed experts per token (10) */
    int32_t ffn;          /* F: routed expert SwiGLU width (640) */
    int32_t shared_ffn;   /* shared expert SwiGLU width (640); 0 = no shared expert */
    int32_t act_dtype;    /* lmoe_dtype of x, y (and of the block's internal activations) */
    int32_t dense_dtype;  /* lmoe_dtype of D, U, Wr and the shared expert */
    int32_t expert_dtype; /* lmoe_dtype of the routed expert records */
    int32_t groups;       /* G: expert groups with their own D/U pair (0 or 1: one pair per layer) */
    /* MXFP4 routed experts: the smallest batch that takes the block-scaled MFMA kernels (CDNA4
     * v_mfma_scale_f32_32x32x64_f8f6f4 with the records as stored and MXFP8 activations).
     * 0 = 96 (the measured crossover against the weight-streaming kernels); -1 = never (batches of
     * 65 .. 383 tokens then take the weight-streaming kernels and larger ones decode the touched
     * records to bf16); values from 1 to 64 count as 65.  Ignored for other expert dtypes. */
    int32_t mx_mfma_min_t;
} lmoe_config;

typedef struct {
    const void* D;        /* [latent][hidden], dense dtype */
    const void* U;        /* [hidden][latent], dense dtype */
    const void* Wr;       /* [n_experts][latent], dense dtype */
    const float* br;      /* [n_experts] fp32 router bias, or NULL for none */
    const void* shared;   /* one packed record (dense dtype, shared_ffn), or NULL iff shared_ffn == 0 */
    const void* experts;  /* n_experts packed records (expert dtype; F32: row-major) */
    const void* Gr;       /* [n_experts][2][hidden] bf16 folded router from lmoe_fold_router, or
                             NULL (ignored for F32 configurations) */
} lmoe_weights;

/* Stages of lmoe_forward, in launch order (for lmoe_forward_opts.stage_events). */
typedef enum {
    LMOE_STAGE_PRENORM = 0,     /* RMSNorm of the fp32 residual into the bf16 block input */
    LMOE_STAGE_D = 1,           /* z = x D^T (with weights->Gr and T <= 64, also the logits) */
    LMOE_STAGE_ROUTER = 2,      /* logits = z Wr^T + br (not recorded when folded into D) */
    LMOE_STAGE_TOPK = 3,        /* top_k + softmax over the kept logits, and the permutation (for
                                   T <= 64 inside the EXPERT_UP launch, not recorded) */
    LMOE_STAGE_PERMUTE = 4,     /* (not recorded: the permutation belongs to the TOPK stage) */
    LMOE_STAGE_EXPERT_UP = 5,   /* SwiGLU gate/up of every segment (shared expert included); for
                                   T <= 64 the routing first */
    LMOE_STAGE_EXPERT_DOWN = 6, /* down projections; for T <= 64 also the weighted merge */
    LMOE_STAGE_COMBINE = 7,     /* weighted merge (T > 64) */
    LMOE_STAGE_U = 8,           /* y = m U^T */
    LMOE_N_STAGES = 9
} lmoe_stage;

typedef struct {
    /* prenorm = 1: x is an fp32 residual stream h [T][hidden]; the block input is
     * bf16(RMSNorm(h)) with unit gain and eps 1e-6 (requires act BF16).  A learned gain g is
     * not an argument: it scales the columns of D (D diag(g)), so a caller folds it into D (and
     * then into the folded router) once; the only difference is where the block input is
     * rounded to bf16 (before the gain instead of after it). */
    int32_t prenorm;
    /* residual = 1: y is fp32 [T][hidden] and is updated in place, y += block output.
     * With prenorm and residual both set, x and y may be the same buffer. */
    int32_t residual;
    /* Optional exports (NULL = skip), all device buffers: */
    float* aux_z;          /* [T][latent] fp32 latent z = x D^T (router input); with G expert
                              groups [T][G*latent], group g's latent in columns g*latent .. */
    int32_t* aux_ids;      /* [T][top_k] chosen experts, ascending id */
    float* aux_w;          /* [T][top_k] routing weights, same order */
    int32_t* aux_offsets;  /* [n_experts + 1] segment starts of the permutation */
    int32_t* aux_perm;     /* [T * top_k] the permutation (see lmoe_permute) */
    /* Optional timing hook: NULL, or an array of 2 * LMOE_N_STAGES hipEvent_t handles
     * (created by the caller; NULL entries are skipped).  Event 2s is recorded on `stream`
     * just before stage s is enqueued and event 2s+1 just after it.  The hook is ignored
     * while `stream` is being captured into a graph. */
    void* const* stage_events;
} lmoe_forward_opts;

/* Bytes of one routed expert record (shared = 0) or of the shared expert record (shared = 1).
 * Returns 0 for an invalid configuration. */
size_t lmoe_expert_record_bytes(const lmoe_config* cfg, int32_t shared);

/* Workspace bytes lmoe_forward needs for T tokens (monotone in T).  MXFP4 layers take the
 * block-scaled MFMA kernels (CDNA4 v_mfma_scale_*_f8f6f4, the records used as stored) from
 * cfg->mx_mfma_min_t tokens (default 96; below it, from 65 tokens, the weight-streaming kernels);
 * the workspace then holds z as MXFP8 plus an MXFP4 residual and H as MXFP8 (about
 * T * (1.56 * latent * groups + 1.03 * top_k * ffn) bytes more).  NVFP4 layers with T >= 384, and
 * MXFP4 layers with T >= 384 when mx_mfma_min_t is -1, decode the records of the experts with
 * tokens to bf16 and the workspace includes n_experts such records (3 * ffn * latent * 2 bytes
 * each).  The result depends on the configuration and T only. */
lmoe_status lmoe_workspace_bytes(const lmoe_config* cfg, int32_t T, size_t* bytes);

/* Workspace bytes lmoe_permute needs for T tokens. */
lmoe_status lmoe_permute_workspace_bytes(const lmoe_config* cfg, int32_t T, size_t* bytes);

/*
 * Expert record packing (a layout step before lmoe_forward; no arithmetic).
 *   shared = 0: n_records routed records (expert dtype); shared = 1: the shared record
 *   (dense dtype, shared_ffn; n_records <= 1).
 *   src: n_records row-major records; dst: the same number of packed records.  src and dst
 *   must not overlap.  F32 configurations return LMOE_ERR_UNSUPPORTED (their records are
 *   read row-major).
 */
lmoe_status lmoe_pack_experts(const lmoe_config* cfg, int32_t shared, const void* src, void* dst, int32_t n_records,
                              void* stream);

/*
 * Router folding (a weight step before lmoe_forward; BF16 dense weights only).  The router
 * logits are linear in the block input: z . Wr^T = x . (Wr D)^T with z = x . D^T.
 * lmoe_fold_router computes G = Wr . D ([n_experts][hidden], fp32 accumulation in ascending
 * latent order; with expert groups, row e of G is Wr[e] . D_{group of e}) and stores it as
 * two bf16 halves, hi = bf16(G) and lo = bf16(G - hi):
 *   Gr [n_experts][2][hidden]  (lmoe_fold_router_bytes(cfg) bytes; must not overlap D or Wr).
 * With weights->Gr set, lmoe_forward computes the logits of batches of up to 64 tokens as
 * x . hi^T + x . lo^T + br in the launch that computes z, one dependent launch fewer than
 * the z-based router.  hi + lo carries G to about 2^-17 relative, the precision the z-based
 * small-batch router keeps for z (a bf16 hi/lo split of the fp32 z).  Larger batches use the
 * z-based router, except with expert groups, where every batch takes its logits from x and
 * the folded router (a GEMM over both halves).  F32 configurations return
 * LMOE_ERR_UNSUPPORTED.
 */
size_t lmoe_fold_router_bytes(const lmoe_config* cfg);
lmoe_status lmoe_fold_router(const lmoe_config* cfg, const void* D, const void* Wr, void* Gr, void* stream);

/*
 * Router (the model-detail page's architecture section: the router selects 10 of the 512
 * experts, Fig. 3 caption).
 *   z   [T][latent] fp32 latent states;
 *   ids [T][top_k] int32 out: the top_k experts of each token, ascending id;
 *   w   [T][top_k] fp32 out: softmax over the selected logits, same order.
 * Uses weights->Wr (dense dtype) and weights->br (may be NULL); other weight pointers are
 * ignored.  ws/ws_bytes: workspace of at least T * n_experts * 4 bytes, where the logits are
 * staged (lmoe_workspace_bytes(cfg, T) is always enough).
 */
lmoe_status lmoe_route(const lmoe_config* cfg, const lmoe_weights* weights, const float* z, int32_t T,
                       int32_t* ids, float* w, void* ws, size_t ws_bytes, void* stream);

/*
 * Token -> expert permutation used to group each expert's tokens into one contiguous
 * segment.  The pages do not describe this step: it is this library's own (the grouping that
 * its expert kernels read), exported so that it can be checked on its own against a stable
 * sort.  Flat slot index f = t*top_k + s.
 *   ids     [T][top_k] int32 in: expert of each slot; the ids of one token must be distinct.
 *   offsets [n_experts + 1] int32 out: offsets[e] = first position of expert e's segment
 *           (exclusive prefix sum of the per-expert counts), offsets[n_experts] = number of
 *           valid slots;
 *   perm    [T*top_k] int32 out: perm[p] = the slot f at position p; inside a segment the
 *           slots are in ascending f (a stable sort, so the result is unique);
 *   inv     [T*top_k] int32 out: inv[f] = p with perm[p] = f.
 * Slots whose id is outside [0, n_experts) are dropped: inv = -1 for them and positions
 * at or after offsets[n_experts] hold -1.  Duplicate ids inside one token give undefined
 * (but in-bounds) contents.
 */
lmoe_status lmoe_permute(const lmoe_config* cfg, const int32_t* ids, int32_t T, int32_t* offsets, int32_t* perm,
                         int32_t* inv, void* ws, size_t ws_bytes, void* stream);

/*
 * The whole block for T tokens.
 *   x [T][hidden] in: act dtype (fp32 when opts->prenorm);
 *   y [T][hidden] out: act dtype, or fp32 accumulated in place when opts->residual.
 * x and y must not overlap, except x == y with prenorm and residual both set.
 * opts may be NULL (plain block, no exports).  ws: lmoe_workspace_bytes(cfg, T) bytes.
 */
lmoe_status lmoe_forward(const lmoe_config* cfg, const lmoe_weights* weights, const void* x, int32_t T, void* y,
                         const lmoe_forward_opts* opts, void* ws, size_t ws_bytes, void* stream);

/*
 * Allocation-free form of lmoe_forward, for callers that cannot allocate device memory or
 * manage a workspace: code being captured into a HIP graph, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments and results as lmoe_forward without ws/ws_bytes: its
 * workspace is a static device array of LMOE_NOALLOC_SCRATCH_BYTES that the library holds on
 * every GPU it runs on (from the loading of its code object until the process ends), found on
 * the first call on each device (the device current on the calling thread, which must be the
 * stream's device).  The call allocates nothing and frees nothing.
 *   - T must need at most LMOE_NOALLOC_SCRATCH_BYTES of workspace (lmoe_workspace_bytes): every
 *     batch of up to 64 tokens at the Edge0-145B shape with bf16, MXFP4 or NVFP4 experts, with
 *     one or 8 expert groups, fits (3.4 MB and 22.2 MB at T = 64); larger requests return
 *     LMOE_ERR_WORKSPACE before anything is enqueued.
 *   - Every call on one GPU uses that GPU's one array, which keeps the last call's contents
 *     (nothing in it needs to start at zero).  Calls on one GPU must therefore be ordered (one
 *     stream, or events between streams): calls that overlap in time on one GPU race and give
 *     undefined results.
 */
#define LMOE_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
lmoe_status lmoe_forward_noalloc(const lmoe_config* cfg, const lmoe_weights* weights, const void* x, int32_t T,
                                 void* y, const lmoe_forward_opts* opts, void* stream);

/* Static text for a status code. */
const char* lmoe_status_str(lmoe_status status);

/* Text of the last error reported by a call on this thread ("" if none). */
const char* lmoe_last_error(void);

/* ABI version: major * 10000 + minor * 100 + patch. */
int32_t lmoe_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LMOE_H */
