/*
 * moe.h -- C ABI of the MI355X (gfx950) sparse-MoE decode layer.
 *
 * The layer (per token t of a decode batch of T tokens, E experts, top_k = k):
 *   logits[t, e] = sum_h W_r[e, h] * x[t, h]  (+ bias[e])
 *   ids[t, 0..k)  = the k largest logits, ordered by (logit descending,
 *                   expert index ascending); ties go to the lower index
 *   w[t, j]       = softmax over all E logits, renormalised over the k chosen
 *   routes r = t*k + j are grouped by expert with a stable counting sort
 *   pass 1: for each unique expert e, each row of gate_up[e] is read once and
 *           applied to every route of e:  g = gate_up[e][i]   . x[t]
 *                                         u = gate_up[e][I+i] . x[t]
 *                                         a[r, i] = silu(g) * u
 *   pass 2: each row of down[e] is read once and applied to every route of e:
 *           y[r, h] = down[e][h] . a[r]
 *   combine: out[t, h] = sum_j w[t, j] * y[t*k + j, h]   (j ascending)
 *
 * Sources (page title, section):
 *  - "MoE Performance Optimization Analysis" (markbaseengine): Root Cause
 *    (router, top-expert selection, experts, combine per layer) and Option 1 /
 *    GPU Router Design (router, selection and dispatch on the device, no host
 *    read and no wait per layer).
 *  - "perf(cpu-moe): dedup experts across the batch in pass 1" (FreeToken
 *    PR #46), commit message and "What this adds": routes grouped by expert
 *    with a counting sort over their ids; pass 1 split by (unique expert, row
 *    block) with the expert's routes as the inner loop; pass 2 (down) per
 *    route, or deduplicated the same way as the follow-up change does.
 *  - "TEXT Generation Optimization Report" (markbaseengine), Phase 1: a whole
 *    forward recorded as one submission with one wait.
 *  The gating function (softmax, top-k, renormalise), SiLU(gate) * up, the
 *  gate/up row split [0, I) / [I, 2I) and the lowest-index tie rule are the
 *  workload's definition; the pages leave them open.
 *
 * Conventions for every entry point:
 *  - Every tensor pointer is a DEVICE pointer owned by the caller.  The
 *    library never allocates, frees or caches device memory; scratch comes
 *    from the caller's workspace `ws` of `ws_bytes` bytes (see
 *    moe_workspace_bytes).  A new workspace is prepared once with
 *    moe_workspace_init, which zeroes its synchronisation words: a front of
 *    fixed size and place (about 256 KiB) that depends on nothing else.
 *    Every call leaves them zero again; the rest of the workspace is
 *    scratch.  So one workspace serves any batch (up to what its ws_bytes
 *    holds) and any layer shape, with any ws_bytes passed per call, as long
 *    as calls that share it are ordered on one stream.
 *  - Batches: 0 <= T <= 65536 tokens per call (MOE_ERR_SHAPE above).
 *  - Calls only enqueue work on `stream` (a hipStream_t; NULL = the null
 *    stream) and return.  They never synchronise or read device memory back,
 *    so they can be recorded into a HIP graph.
 *  - Layout is row-major and contiguous.  Activations, logits, weights of the
 *    combine and outputs are fp32; expert weights are fp32, bf16, OCP fp8
 *    E4M3 with fp32 scales per 128x128 block, or OCP MXFP4; the router is
 *    fp32 or bf16.
 *  - The status covers host-side validation and launch errors only.  A
 *    device fault shows up at the caller's next synchronisation.  Inputs must
 *    be finite: NaN or Inf give an unspecified routing.
 *  - T == 0 is a no-op that returns MOE_OK.
 *  - Threads: entry points may be called from several host threads at once.
 *    Calls that share a workspace, or a stream, must not overlap: order them
 *    on one stream, issued by one thread at a time.  For batches of 128
 *    tokens or more whose experts run partly on the matrix cores, the
 *    library keeps one side stream and two events per (device, caller
 *    stream) pair, created on the first such call made outside a graph
 *    capture and kept until the process ends; a call enqueues its whole
 *    fork/join sequence under a lock.  Apart from that and the device's
 *    compute-unit count, the library holds no state between calls.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_ARG = 1,         /* NULL pointer, negative size, k < 1 or k > E ... */
    MOE_ERR_SHAPE = 2,       /* size limits or divisibility (see below)       */
    MOE_ERR_DTYPE = 3,       /* unknown dtype or combination                   */
    MOE_ERR_WORKSPACE = 4,   /* ws NULL or smaller than required               */
    MOE_ERR_HIP = 5,         /* a HIP launch reported an error                 */
    MOE_ERR_UNSUPPORTED = 6, /* valid request the library does not implement   */
    MOE_ERR_ALIGN = 7        /* a pointer is not 16-byte aligned               */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3 = 2, MOE_MXFP4 = 3, MOE_Q4_0 = 4 } moe_dtype;

/* One MoE layer.  Limits: 1 <= E <= 1024, 1 <= top_k <= min(E, 32);
 * H, I >= 1 with H, I multiples of 4 (fp32), 8 (bf16), 128 (fp8) or 32
 * (MXFP4, q4_0), and at most 512 16-byte chunks per weight row (H, I <= 2048
 * fp32, 4096 bf16, 8192 fp8, 16384 MXFP4 and q4_0).  Weight pointers must be 16-byte
 * aligned.
 *
 * MXFP4 expert weights (OCP microscaling): E2M1 codes, two per byte with the
 * even element in the low nibble (a row of K elements is K/2 bytes), and one
 * E8M0 scale byte, 2^(s - 127), per 32 consecutive elements of a row:
 * s_gate_up uint8 [E, 2I, H/32], s_down uint8 [E, H, I/32].  The router
 * stays fp32 or bf16.
 *
 * q4_0 expert weights (the q4_0 format of the pages' list of formats on the
 * pass-1 dot product: blocks of 32 consecutive elements of a row, one
 * IEEE binary16 scale d per block, 4-bit codes q, value (q - 8) * d): a
 * block is 16 code bytes, element j < 16 in the low nibble of byte j and
 * element j + 16 in its high nibble (a row of K elements is K/2 bytes); the
 * scales sit in their own arrays, binary16 bit patterns, 2-byte aligned:
 * s_gate_up uint16 [E, 2I, H/32], s_down uint16 [E, H, I/32].  On the
 * matrix cores (scale arrays 4-byte aligned) the codes minus 8 are exact bf16
 * operands below 128 tokens, each k-step's sums scaled by the rows' scales;
 * from 128 tokens each operand is (code - 8) * scale rounded to bf16 once.
 *
 * Matrix cores: in a call of 16 or more tokens, an expert that holds
 * moe_mfma_min_routes() routes or more (5 below 128 tokens, 4 from 128) runs,
 * in moe_layer_fwd and moe_stack_fwd when the call's largest expert holds
 * moe_mfma_hot_routes() routes or more (8 below 128 tokens), both passes as
 * bf16 MFMA products with fp32 accumulation (the activations
 * and the decoded weights rounded to bf16; decoded MXFP4 weights are exact in
 * bf16) when the experts are bf16, fp8, MXFP4 or q4_0 with H and I multiples
 * of 128 (MXFP4 and q4_0 also need 4-byte aligned scale arrays; q4_0 operands
 * as described above), unless the flags ask
 * for MOE_NO_MFMA or the per-route walk.  Every other segment runs on the
 * GEMV kernels (fp32 accumulation of exactly decoded weights). */
typedef struct {
    int32_t E, top_k, H, I;
    int32_t router_dtype;     /* MOE_F32 or MOE_BF16                          */
    int32_t expert_dtype;     /* MOE_F32, MOE_BF16, MOE_FP8_E4M3, MOE_MXFP4 or MOE_Q4_0 */
    const void *w_router;     /* [E, H]                                       */
    const void *w_gate_up;    /* [E, 2I, H]: rows [0, I) gate, [I, 2I) up     */
    const void *w_down;       /* [E, H, I]                                    */
    const void *s_gate_up;    /* fp8: float [E, 2I/128, H/128]; MXFP4: uint8, q4_0: uint16 [E, 2I, H/32] */
    const void *s_down;       /* fp8: float [E, H/128, I/128]; MXFP4: uint8, q4_0: uint16 [E, H, I/32]   */
    const float *router_bias; /* [E] added to the logits, or NULL             */
} moe_layer_t;

/* flags */
enum {
    MOE_WALK_DEDUP = 0,        /* pass 1 and pass 2 once per unique expert     */
    MOE_WALK_PER_ROUTE = 1,    /* every route reads its expert itself          */
    MOE_WALK_DEDUP_PASS1 = 2,  /* pass 1 per unique expert, pass 2 per route   */
    MOE_WALK_MASK = 0xF,
    MOE_ACCUM_RESIDUAL = 1 << 4, /* out = x + MoE(...) (x = the layer input)   */
    MOE_RMSNORM_IN = 1 << 6,     /* normalise x (eps 1e-6, gamma 1) first       */
    MOE_NO_MFMA = 1 << 7         /* keep every segment on the GEMV path         */
};

/* Bytes of workspace needed for up to max_tokens tokens (max_tokens >= 0).
 * Returns 0 if the layer description is invalid. */
size_t moe_workspace_bytes(const moe_layer_t *layer, int32_t max_tokens);

/* Routes an expert must hold in a call of T tokens for its segment to run on
 * the matrix cores (bf16 MFMA: the activations rounded to bf16, fp32
 * accumulation; the GEMV kernels keep fp32 activations), or 0 when no
 * segment of such a call does: weights not bf16 / fp8 / MXFP4 with H and I
 * multiples of 128, T below 16, activation rows of 2 GiB or more,
 * MOE_NO_MFMA or the per-route walk in flags.  Which segments run where
 * decides the rounding of their results, so callers and tests can tell.
 * Host only (no device work); -1 for an invalid layer, T < 0 or an unknown
 * walk in flags.  The thresholds: 5 routes below 128 tokens, 4 from 128
 * tokens (the workload definition leaves "dense enough" open; these are
 * measured crossovers). */
int32_t moe_mfma_min_routes(const moe_layer_t *layer, int32_t T, uint32_t flags);

/* In moe_layer_fwd and moe_stack_fwd (whose own sort knows the largest
 * expert), the segments of moe_mfma_min_routes() routes or more take the
 * MFMA path only if the call's largest expert holds this many routes or
 * more: 8 below 128 tokens (an MFMA launch with a few small experts costs
 * more than it saves), moe_mfma_min_routes() from 128; 0 when no segment
 * does.  moe_expert_fwd, given its routing, applies moe_mfma_min_routes()
 * alone.  Host only; -1 as for moe_mfma_min_routes. */
int32_t moe_mfma_hot_routes(const moe_layer_t *layer, int32_t T, uint32_t flags);

/* Zero the synchronisation words at the front of a workspace sized for up to
 * max_tokens tokens (one small fill kernel on `stream`; no memset, so it can
 * be recorded in a graph).  Call once after allocating ws, before the first
 * call that uses it. */
moe_status moe_workspace_init(const moe_layer_t *layer, int32_t max_tokens, void *ws, size_t ws_bytes,
                              void *stream);

/* Router and selection.  Either x [T, H] (logits computed on the device from
 * W_r and router_bias) or logits_in [T, E] (selection fed with given logits)
 * must be non-NULL; logits_in wins if both are.  Writes topk_ids [T, k]
 * (int32) and topk_w [T, k] (fp32) and, if non-NULL, logits_out [T, E].
 * With x, ws (moe_workspace_bytes(layer, T) bytes, initialised) is required;
 * with logits_in it may be NULL. */
moe_status moe_route(const moe_layer_t *layer, const float *x, const float *logits_in, int32_t T,
                     float *logits_out, int32_t *topk_ids, float *topk_w, void *ws, size_t ws_bytes,
                     void *stream);

/* Stable counting sort of the T*k routes (r = t*k + j) by expert id.
 * counts [E]; offsets [E+1] exclusive prefix sum (offsets[E] = T*k);
 * sorted_routes [T*k]: routes of expert 0, then 1, ..., each ascending;
 * uniq [E]: experts with a nonzero count, ascending (first n_uniq entries);
 * n_uniq [1].  An id outside [0, E) sets *n_uniq = -1 and leaves the other
 * outputs unspecified (nothing is written out of bounds). */
moe_status moe_sort(const int32_t *topk_ids, int32_t T, int32_t k, int32_t E, int32_t *counts, int32_t *offsets,
                    int32_t *sorted_routes, int32_t *uniq, int32_t *n_uniq, void *stream);

/* Experts and combine for a given routing (the outputs of moe_route and
 * moe_sort on the same ids).  x [T, H] is the expert input; out [T, H] is
 * overwritten (flags MOE_ACCUM_RESIDUAL: out = x + combine).  The walk arm
 * comes from flags & MOE_WALK_MASK; all arms give bitwise the same output
 * when no segment takes the MFMA path.  out may alias x.  A routing the sort
 * rejected (*n_uniq < 0, read on the device) runs no expert work and leaves
 * out untouched. */
moe_status moe_expert_fwd(const moe_layer_t *layer, const float *x, int32_t T, const int32_t *topk_ids,
                          const float *topk_w, const int32_t *counts, const int32_t *offsets,
                          const int32_t *sorted_routes, const int32_t *uniq, const int32_t *n_uniq, float *out,
                          uint32_t flags, void *ws, size_t ws_bytes, void *stream);

/* The whole layer: [RMSNorm] -> router -> selection -> sort -> pass 1 ->
 * pass 2 -> combine [-> + x], all on the device.  out may alias x.  After the
 * call (once the stream reaches it) the first 16 bytes of ws hold int32
 * {n_uniq, T*k, max routes of one expert, 0}. */
moe_status moe_layer_fwd(const moe_layer_t *layer, const float *x, int32_t T, float *out, uint32_t flags,
                         void *ws, size_t ws_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the layer
 * exactly as moe_layer_fwd computes it, bit for bit, with its scratch in a
 * device array that the library holds instead of a caller workspace:
 * MOE_STATIC_SCRATCH_BYTES (16 MiB) on each GPU the library runs on, kept
 * until the process ends.  The caller passes inputs and outputs only.  A
 * batch whose layer needs more scratch than that
 * (moe_workspace_bytes(layer, T) > MOE_STATIC_SCRATCH_BYTES, e.g. beyond
 * 159 tokens for E=256, top_k=8, H=2048, I=768) is refused with
 * MOE_ERR_WORKSPACE before anything is enqueued.  No memory is allocated:
 * the first call on a device looks the array's address up and clears its
 * synchronisation words with a fill kernel on `stream`, and every call
 * leaves them clear again.  All calls on one GPU share the array, which
 * keeps the last call's contents, so calls that overlap on one GPU race:
 * order them on one stream.  The matrix-core segments of large batches run
 * in order on `stream` (no side stream). */
#define MOE_STATIC_SCRATCH_BYTES ((size_t)16 << 20)
moe_status moe_layer_fwd_static(const moe_layer_t *layer, const float *x, int32_t T, float *out, uint32_t flags,
                                void *stream);

/* moe_layer_fwd with per-stage timing: events[s] (hipEvent_t, created by
 * the caller with timing enabled) is recorded on `stream` before stage s and
 * events[MOE_N_STAGES] after the last, for the stages
 *   0 routing (RMSNorm, router, selection, sort), 1 pass 1 GEMV segments,
 *   2 pass 1 MFMA segments, 3 pass 2 MFMA segments, 4 pass 2 GEMV segments
 *   (with the combine for batches up to 64 tokens whose down rows take 32
 *   or 64 lanes: not MXFP4 or q4_0 rows with I not a multiple of 1024),
 *   5 combine.
 * A stage that does not run for this call takes no time between its two
 * events.  events == NULL behaves as moe_layer_fwd; a NULL entry is
 * MOE_ERR_ARG.  For kernel timing in benchmarks; the extra event records
 * make it unsuited to graph capture. */
enum { MOE_N_STAGES = 6 };
moe_status moe_layer_fwd_events(const moe_layer_t *layer, const float *x, int32_t T, float *out, uint32_t flags,
                                void *ws, size_t ws_bytes, void *stream, void *const *events);

/* Device addresses, inside a workspace that moe_layer_fwd used for T tokens,
 * of the routing that call computed (valid once the stream has reached it,
 * until the workspace is reused): topk_ids [T, k], topk_w [T, k],
 * counts [E], offsets [E+1], sorted_routes [T*k], uniq [E], n_uniq [1].
 * Any output pointer may be NULL.  For expert-usage telemetry and tests. */
moe_status moe_layer_routing(const moe_layer_t *layer, int32_t T, void *ws, size_t ws_bytes, int32_t **topk_ids,
                             float **topk_w, int32_t **counts, int32_t **offsets, int32_t **sorted_routes,
                             int32_t **uniq, int32_t **n_uniq);

/* Expert-usage telemetry: hist[e] += counts[e] for e < E, on `stream`, with
 * hist a caller-owned device array of E uint64 counters (8-byte aligned) that
 * accumulates across calls; nothing is added when *n_uniq < 0 (the sort
 * rejected the routing).  counts and n_uniq are the outputs of moe_sort, or
 * the addresses moe_layer_routing returns after a moe_layer_fwd call, so a
 * recorded graph can add each layer's usage after its forward.
 * "MoE Performance Optimization Analysis", Option 3 (expert caching) and
 * Phase 3: track per-layer expert usage.  Errors: NULL pointer or E < 1
 * (MOE_ERR_ARG), E > 1024 (MOE_ERR_SHAPE), misaligned hist (MOE_ERR_ALIGN). */
moe_status moe_expert_usage(const int32_t *counts, const int32_t *n_uniq, int32_t E, uint64_t *hist,
                            void *stream);

/* A stack of layers, h_{l+1} = h_l + MoE_l(RMSNorm(h_l)) for l = 0 ..
 * n_layers - 1 with h_0 = x and out = h_{n_layers}: the same result, bit for
 * bit, as n_layers moe_layer_fwd calls with MOE_RMSNORM_IN |
 * MOE_ACCUM_RESIDUAL, in one launch fewer per layer: the combine and residual
 * of layer l run inside the routing launch of layer l + 1, which forms its
 * input rows from layer l's outputs (only the last layer launches a combine).
 * "TEXT Generation Optimization Report" (markbaseengine), Phase 2: fuse the
 * operations around each layer to cut dispatches per token.
 * layers: n_layers >= 1 descriptions of one shape (E, top_k, H, I and dtypes
 * equal; weights may differ), else MOE_ERR_SHAPE.  flags: a walk arm and
 * MOE_NO_MFMA; MOE_RMSNORM_IN and MOE_ACCUM_RESIDUAL are implied.  out may
 * alias x.  ws: moe_stack_workspace_bytes(layers, max_tokens) bytes, prepared
 * once with moe_stack_workspace_init (it zeroes two fixed fronts of
 * synchronisation words); as for a layer workspace, calls on it may pass
 * any batch it holds. */
size_t moe_stack_workspace_bytes(const moe_layer_t *layer, int32_t max_tokens);
moe_status moe_stack_workspace_init(const moe_layer_t *layer, int32_t max_tokens, void *ws, size_t ws_bytes,
                                    void *stream);
moe_status moe_stack_fwd(const moe_layer_t *layers, int32_t n_layers, const float *x, int32_t T, float *out,
                         uint32_t flags, void *ws, size_t ws_bytes, void *stream);

/* Static text for a status code. */
const char *moe_status_str(moe_status status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
