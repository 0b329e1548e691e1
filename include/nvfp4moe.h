/*
 * nvfp4moe.h -- C ABI of the MI355X (gfx950) NVFP4 weight-only MoE / projection library.
 *
 * The operations follow three public pull-request pages of the 1Cat-vLLM project.
 *   "[Kernel][SM70] Improve Qwen3.8 no-MTP concurrency", sections "Scope and related PRs", "Test
 *   Result" and "Latest grouped-MoE screen": native NVFP4 weights with FP16 activations. Expert
 *   dispatch runs an expert-grouped W13 with fused SiLU(gate)*up, then a grouped W2 and its
 *   reduction. Both reuse one integer routing plan, so planning is not repeated. W13 has two
 *   physical layouts. Metadata checks fail closed.
 *   "[SM70][Draft] Extend Qwen3.8 DFlash2 concurrency paths", sections "Purpose" and "TP4-only
 *   NVFP4 verifier follow-up": the dense "QPN" NVFP4 projection for small M, and its batch
 *   invariance (an M-row result equals the concatenated 8-row results, bitwise).
 *
 * Number format (NVFP4). The pages name NVFP4 but print no layout. This library uses the
 * standard one, the plainest reading:
 *   codes   uint8  [groups][rows][k/2]   two OCP E2M1 codes per byte; even k in the low nibble
 *   scales  uint8  [groups][rows][k/16]  one OCP E4M3FN byte per 16-element K-block
 *   global  float  [groups]              one FP32 global scale per group (per expert, or 1 for a
 *                                         dense weight)
 *   w[g][n][k] = e2m1(code) * e4m3(scale[g][n][k/16]) * global[g]
 * Activations and outputs are IEEE binary16 (passed as uint16_t bit patterns); accumulation is FP32.
 *
 * Conventions for every entry point:
 *   - Every pointer argument except `w` descriptors and the stream is a DEVICE pointer. The
 *     nvfp4_weights descriptor itself is read on the host during the call; the pointers inside it
 *     are device pointers.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream). Calls only enqueue work
 *     on it: no host synchronisation, no device allocation, no device-to-host copy. Every call can
 *     therefore be captured in a HIP graph.
 *   - The caller allocates and owns every buffer (plan, workspace, outputs). The library keeps no
 *     pointer after a call returns and holds no mutable global state (except the static device
 *     array of nvfp4_moe_layer_noalloc), so calls from several host threads on different streams
 *     are safe. Two calls that write the same buffer must be ordered
 *     by the caller (for example, the same stream).
 *   - Errors fail closed: a nonzero status is returned, nothing is enqueued, and no output is
 *     touched. Status codes are NVFP4_* below; nvfp4_status_str() names them. Every argument and
 *     every launch's resources (grid, LDS) are checked before the first launch of a call, so the
 *     one exception is NVFP4_ERR_LAUNCH from a call that enqueues several kernels: the runtime may
 *     reject a later launch after earlier ones were enqueued, and the outputs are then undefined.
 *   - M = 0 is a successful no-op.
 *   - Arithmetic does not depend on M or on other tokens. A token's output is bitwise the same
 *     whether it runs alone or in any batch (for the MoE: with the same routing row and weights).
 */
#ifndef NVFP4MOE_H
#define NVFP4MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NVFP4_ABI_VERSION 1

enum {
    NVFP4_OK = 0,
    NVFP4_ERR_NULL = 1,        /* a required pointer is NULL                                   */
    NVFP4_ERR_SHAPE = 2,       /* inconsistent or out-of-range sizes                           */
    NVFP4_ERR_ALIGN = 3,       /* a pointer is not 16-byte aligned                              */
    NVFP4_ERR_WORKSPACE = 4,   /* plan or workspace buffer smaller than the *_bytes() size      */
    NVFP4_ERR_UNSUPPORTED = 5, /* a valid shape for which no kernel is built (see each call)    */
    NVFP4_ERR_LAUNCH = 6       /* the HIP runtime rejected a launch                             */
};

/* A quantized weight tensor: `groups` matrices of `rows` x `k`. */
typedef struct nvfp4_weights {
    const uint8_t *codes;       /* device, [groups][rows][k/2], 16-byte aligned                */
    const uint8_t *scales;      /* device, [groups][rows][k/16], 8-byte aligned                */
    const float *global_scale;  /* device, [groups]                                            */
    int32_t groups, rows, k;
} nvfp4_weights;

/* A channel-FP8 weight tensor (the "QPN8" format): `rows` x `k` E4M3FN bytes and one FP32 scale
 * per row (output channel). */
typedef struct fp8_channel_weights {
    const uint8_t *codes;          /* device, [rows][k] E4M3FN bytes, 16-byte aligned            */
    const float *channel_scale;    /* device, [rows]                                             */
    int32_t rows, k;
} fp8_channel_weights;

/* ABI version of the loaded library (NVFP4_ABI_VERSION). A caller checks it before use
 * ("native ABI capability check", DFlash2 page, "Purpose"). */
int nvfp4_abi_version(void);

/* Static, NUL-terminated name of a status code. Never NULL. */
const char *nvfp4_status_str(int status);

/* ---------------------------------------------------------------------------------------------
 * Routing plan (the one integer plan that W13 and the grouped W2 share, no-MTP page, "Scope and
 * related PRs").
 *
 * Input topk_ids int32 [M][topk]. Pair p = t*topk + k. An id in [0, E) routes the pair to that
 * expert. -1 means "no expert", and the pair is skipped. Any other id is also skipped and is
 * counted in the plan's bad-id word. The plan is a stable counting sort of the valid pairs by
 * expert (ties by ascending p), so it is unique and the device result is bit-exact.
 *
 * Plan layout (int32 words, from the start of `plan`; P = M*topk, A = min(E, P),
 * T = A + ceil(P/16)):
 *   [0] n_valid  [1] n_active  [2] n_bad  [3] n_tiles  [4] M  [5] topk  [6] E  [7] 16 (tile rows)
 *   [8..15] reserved
 *   counts[E]  offsets[E+1]  active[A]  tile_expert[T]  tile_row0[T]  tile_base[T]  tile_rows[T]
 *   tile_pair[T][16]  sorted_pair[P]  pos_of_pair[P]  pair_expert[P]
 *   followed by internal scratch when P > 1024.
 * Within each array only the first n_valid / n_active / n_tiles entries are defined. pos_of_pair[p]
 * is the bucket-order row of pair p, or -1 if the pair was skipped; pair_expert[p] is its expert,
 * or -1. Active experts are in
 * ascending id order, and row tiles of 16 rows are in (expert, row0) order. Row tile t covers
 * bucket rows tile_base[t] = offsets[e] + tile_row0[t] .. + tile_rows[t] - 1 of its expert e;
 * tile_pair[t][r] is the pair of its row r (undefined for r >= tile_rows[t]). These are redundant with
 * sorted_pair; they let a kernel reach a tile's rows with one dependent load.
 *
 * The plan stays valid until the caller overwrites it. W13 and W2 only read it, and must be given
 * the same M, topk and E. They take no plan size: the buffer must be one that nvfp4_moe_plan (or a
 * call that builds the plan) wrote for that M, topk and E, else their reads are undefined.
 * Requirements: 1 <= topk <= 32, 1 <= E <= 4096, M*topk <= 2^26.
 * --------------------------------------------------------------------------------------------- */
size_t nvfp4_moe_plan_bytes(int32_t M, int32_t topk, int32_t E);
int nvfp4_moe_plan(const int32_t *topk_ids, int32_t M, int32_t topk, int32_t E,
                   void *plan, size_t plan_bytes, void *stream);

/* ---------------------------------------------------------------------------------------------
 * Router fused with the plan (the "router" among the fused MoE parts, no-MTP page, "Scope and
 * related PRs"; the pages print no formula, so this is the plain reading).
 *   logits        fp32 [M][E]      router logits
 *   topk_ids      int32 [M][topk]  output: token t's experts, slot k = its k-th largest logit
 *   topk_weights  fp32 [M][topk]   output: softmax of the selected logits,
 *                                  w[t][k] = exp(l_k - l_0) / sum_j exp(l_j - l_0), FP32
 *   plan          as for nvfp4_moe_plan; the result is the plan of the ids written here
 * Selection order: larger logit first; equal logits (+0 and -0 are equal) in ascending expert id;
 * a NaN logit ranks below every number. The ids are exact (comparisons only). Non-finite selected
 * logits make the weights NaN by IEEE rules (for example l_0 = +inf gives inf - inf).
 * Requirements: 1 <= topk <= min(E, 32), E <= 4096, M*topk <= 2^26; logits, ids, weights 4-byte
 * aligned, plan 16-byte aligned. With M*topk <= 1024 and E <= 1024 routing and planning are one
 * launch.
 * --------------------------------------------------------------------------------------------- */
int nvfp4_moe_route(const float *logits, int32_t M, int32_t E, int32_t topk, int32_t *topk_ids,
                    float *topk_weights, void *plan, size_t plan_bytes, void *stream);

/* ---------------------------------------------------------------------------------------------
 * Grouped W13 with fused SwiGLU (the expert-grouped W13 with SiLU fused, no-MTP page, "Scope and
 * related PRs").
 *   x    fp16 [M][K]          activations (K = w13->k)
 *   w13  groups = E, rows = 2I, k = K
 *        layout 0: gate rows [0, I), up rows [I, 2I)
 *        layout 1: interleaved, row 2i is gate i and row 2i+1 is up i
 *        (the page's "same-split W13 in both physical layouts", "Test Result")
 *   h    fp16 [M*topk][I]      output, in bucket order: row j is pair sorted_pair[j]
 * For bucket row j with pair p = (t, k) and expert e:
 *   g = global[e] * sum_k x[t,k] * e2m1*e4m3 (gate row),  u = likewise (up row),
 *   h[j][i] = fp16_rne( silu(g) * u ),  silu(g) = g / (1 + exp(-g)),  all FP32.
 * Each active expert's weights are read once, for all of its pairs. Rows j >= n_valid are not
 * written.
 * Requirements: K % 128 == 0 and K <= 2048; I % 16 == 0; x, h, codes 16-byte aligned.
 * --------------------------------------------------------------------------------------------- */
int nvfp4_moe_w13_swiglu(const void *plan, int32_t M, int32_t topk, int32_t E,
                         const uint16_t *x, const nvfp4_weights *w13, int32_t layout,
                         uint16_t *h, void *stream);

/* ---------------------------------------------------------------------------------------------
 * Routing plan and grouped W13 + SwiGLU in one call: the results of nvfp4_moe_plan(topk_ids, ...,
 * plan) followed by nvfp4_moe_w13_swiglu(plan, ...), bit for bit (the plan is built once and both
 * W13 and W2 read it, so the layer plans once: no-MTP page, "Scope and related PRs").
 *   topk_ids, plan, plan_bytes   as for nvfp4_moe_plan (plan is written: W2 takes it afterwards)
 *   x, w13, layout, h            as for nvfp4_moe_w13_swiglu
 * With M*topk <= 256, E <= 1024 and the decode (non-prefill) regime, it is one launch: every W13
 * block builds the plan of the ids in LDS and one block writes the plan buffer. Otherwise it
 * enqueues the plan and the W13 launch. Requirements: those of the two calls (K % 128 == 0,
 * K <= 2048, I % 16 == 0). Errors: those of the two calls, all checked before anything is
 * enqueued; M = 0 is an OK no-op.
 * --------------------------------------------------------------------------------------------- */
int nvfp4_moe_plan_w13_swiglu(const int32_t *topk_ids, int32_t M, int32_t topk, int32_t E,
                              void *plan, size_t plan_bytes, const uint16_t *x,
                              const nvfp4_weights *w13, int32_t layout, uint16_t *h, void *stream);

/* ---------------------------------------------------------------------------------------------
 * Grouped W2 with the top-k-weighted reduction fused in (no-MTP page, "Scope and
 * related PRs").
 *   h             fp16 [M*topk][I]  W13 output in bucket order
 *   w2            groups = E, rows = K, k = I
 *   topk_weights  fp32 [M][topk]    used exactly as given (no renormalisation)
 *   out           fp16 [M][K]       every element is written
 *   ws            device workspace of at least nvfp4_moe_w2_workspace_bytes(M, topk, K) bytes,
 *                 contents ignored on entry (FP32 per-pair results, row p = t*topk + k)
 * y[j][n] = global[e] * sum_i dq(W2_e)[n][i] * h[j][i], in FP32 with no intermediate rounding. Then
 *   out[t][n] = fp16_rne( s ),  s = 0;  for k = 0..topk-1 with a valid id: s = fmaf(w[t][k], y[pos][n], s)
 * This is slot order. A token with no valid slot gets +0.
 * Requirements: I % 128 == 0 and I <= 2048; K % 64 == 0; h, out, codes 16-byte aligned.
 * --------------------------------------------------------------------------------------------- */
size_t nvfp4_moe_w2_workspace_bytes(int32_t M, int32_t topk, int32_t K);
int nvfp4_moe_w2_reduce(const void *plan, int32_t M, int32_t topk, int32_t E,
                        const uint16_t *h, const nvfp4_weights *w2, const float *topk_weights,
                        uint16_t *out, void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------------------------
 * The whole MoE layer in one call: routing plan, grouped W13 + SwiGLU, grouped W2 and the
 * slot-order reduction (no-MTP page, "Latest grouped-MoE screen", which times grouped W13 and
 * grouped W2 together as one complete call). The results are bitwise those of
 * nvfp4_moe_plan_w13_swiglu followed by nvfp4_moe_w2_reduce with the same arguments; one host call
 * enqueues every launch.
 *   topk_ids, M, topk, E   as for nvfp4_moe_plan
 *   x, w13, layout         as for nvfp4_moe_w13_swiglu (K = w13->k, I = w13->rows / 2)
 *   w2                     groups = E, rows = K, k = I
 *   topk_weights, out      as for nvfp4_moe_w2_reduce
 *   ws                     device workspace, at least nvfp4_moe_layer_workspace_bytes(M, topk, E, K,
 *                          I) bytes, 16-byte aligned, contents ignored on entry. On return it holds
 *                          the plan at byte 0 (nvfp4_moe_plan_bytes(M, topk, E) bytes, the layout of
 *                          nvfp4_moe_plan), h (fp16 [M*topk][I]) at the next multiple of 256 bytes,
 *                          and the W2 workspace after that, also at a multiple of 256. h is in bucket
 *                          order, except on the pair-major path for small batches (4*M*topk <= E,
 *                          M*topk <= 256 and E <= 1024): there row p = t*topk + k holds pair p's h
 *                          (rows of skipped pairs are unspecified), W13 takes its rows straight from
 *                          topk_ids and W2 reads the ids and that h, so no load waits for the plan.
 * Requirements: K % 128 == 0, K <= 2048, I % 128 == 0, I <= 2048, 1 <= topk <= 32, E <= 4096;
 * topk_ids and topk_weights 4-byte aligned; x, out and codes 16-byte aligned. Errors: those of
 * the calls it replaces, all checked before anything is enqueued; M = 0 is an OK no-op.
 * --------------------------------------------------------------------------------------------- */
size_t nvfp4_moe_layer_workspace_bytes(int32_t M, int32_t topk, int32_t E, int32_t K, int32_t I);
int nvfp4_moe_layer(const int32_t *topk_ids, int32_t M, int32_t topk, int32_t E, const uint16_t *x,
                    const nvfp4_weights *w13, int32_t layout, const nvfp4_weights *w2,
                    const float *topk_weights, uint16_t *out, void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------------------------
 * nvfp4_moe_layer without a caller workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc). The call
 * itself allocates nothing: the plan, h and the W2 workspace live in a static device array of
 * NVFP4_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on until the process
 * ends. Arguments, results and requirements are those of nvfp4_moe_layer; the output is bitwise
 * the same. A shape whose nvfp4_moe_layer_workspace_bytes(M, topk, E, K, I) exceeds the array
 * returns NVFP4_ERR_WORKSPACE with nothing enqueued (about 100 tokens at 512 experts, top-10,
 * K = 2048, I = 512). No part of the array needs to start at zero, and every call rewrites what it
 * reads.
 * Every call on one GPU shares that GPU's array: two calls that can overlap on one GPU (different
 * streams, or different host threads without ordering) race and give undefined results; calls on
 * one stream are ordered and safe.
 * --------------------------------------------------------------------------------------------- */
#define NVFP4_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
int nvfp4_moe_layer_noalloc(const int32_t *topk_ids, int32_t M, int32_t topk, int32_t E, const uint16_t *x,
                            const nvfp4_weights *w13, int32_t layout, const nvfp4_weights *w2,
                            const float *topk_weights, uint16_t *out, void *stream);

/* ---------------------------------------------------------------------------------------------
 * Shared expert and shared gate (the "shared gate" among the fused MoE parts, no-MTP page, "Scope
 * and related PRs"; no formula is printed, so this is the plain reading): a dense NVFP4 gated MLP
 * on every token, scaled by sigmoid(x . g) and added to the routed output.
 *   nvfp4_moe_shared_expert: x fp16 [M][K]; w13 groups = 1, rows = 2I, k = K (layouts as for
 *     nvfp4_linear_swiglu); w2 groups = 1, rows = K, k = I; gate fp16 [K];
 *     h fp16 [M][I] (scratch, the gated MLP's h), shared_y FP32 [M][K] = W2 h (unrounded, global
 *     scale applied), shared_sigma FP32 [M] = 1 / (1 + exp(-sum_k x[m][k] gate[k])).
 *     Requirements: K % 128 == 0, K <= 16384, I % 128 == 0, I <= 32768; x, h, shared_y 16-byte
 *     aligned.
 *   nvfp4_moe_w2_reduce_shared: nvfp4_moe_w2_reduce with the shared expert as one more slot after
 *     the routed ones: s = (routed fmaf chain); s = fmaf(shared_sigma[t], shared_y[t][n], s);
 *     out = fp16_rne(s). shared_y 16-byte aligned.
 * --------------------------------------------------------------------------------------------- */
int nvfp4_moe_shared_expert(const uint16_t *x, int32_t M, const nvfp4_weights *w13, int32_t layout,
                            const nvfp4_weights *w2, const uint16_t *gate, uint16_t *h, float *shared_y,
                            float *shared_sigma, void *stream);
int nvfp4_moe_w2_reduce_shared(const void *plan, int32_t M, int32_t topk, int32_t E, const uint16_t *h,
                               const nvfp4_weights *w2, const float *topk_weights, const float *shared_y,
                               const float *shared_sigma, uint16_t *out, void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------------------------
 * The same shared expert and gate run inside the routed launches (the "shared gate" among the
 * fused MoE parts, no-MTP page, "Scope and related PRs"): its rows join the routed W13 and W2
 * launches as extra tiles, so it adds no launches of its own. Results are bitwise those of
 * nvfp4_moe_w13_swiglu + nvfp4_moe_shared_expert, and of nvfp4_moe_w2_reduce_shared.
 *   nvfp4_moe_w13_swiglu_with_shared: nvfp4_moe_w13_swiglu's arguments, plus shared_w13
 *     (groups = 1, rows = 2Is, k = K, same layout), gate fp16 [K], and the outputs shared_h fp16
 *     [M][Is] and shared_sigma FP32 [M] (as in nvfp4_moe_shared_expert).
 *   nvfp4_moe_w2_reduce_with_shared: nvfp4_moe_w2_reduce's arguments, plus shared_h (from the call
 *     above), shared_w2 (groups = 1, rows = K, k = Is), shared_sigma, and shared_y FP32 [M][K],
 *     scratch that the call may overwrite with the shared expert's unrounded output.
 *     out = fp16_rne(fmaf(shared_sigma[t], y_shared[t][n], routed slot chain)).
 * Requirements: those of the routed calls (K <= 2048 and I <= 2048 among them); Is % 16 == 0
 * (W13) and Is % 128 == 0, Is <= 32768 (W2); shared_h, shared_y 16-byte aligned; gate 2-byte
 * aligned. The one-launch form needs Is == I, a 16-byte
 * aligned gate and the streaming (not the prefill) regime; otherwise the call runs the shared
 * expert's own launches after the routed one, with the same results.
 * --------------------------------------------------------------------------------------------- */
int nvfp4_moe_w13_swiglu_with_shared(const void *plan, int32_t M, int32_t topk, int32_t E, const uint16_t *x,
                                     const nvfp4_weights *w13, int32_t layout, uint16_t *h,
                                     const nvfp4_weights *shared_w13, const uint16_t *gate, uint16_t *shared_h,
                                     float *shared_sigma, void *stream);
/* nvfp4_moe_plan_w13_swiglu_with_shared: nvfp4_moe_plan followed by
 * nvfp4_moe_w13_swiglu_with_shared, bit for bit, as nvfp4_moe_plan_w13_swiglu is for the routed
 * call: topk_ids, plan and plan_bytes as for nvfp4_moe_plan, the rest as for
 * nvfp4_moe_w13_swiglu_with_shared. One launch when that call's one-launch form applies and
 * M*topk <= 256, E <= 1024; otherwise the plan is enqueued first. Errors: those of the two calls,
 * all checked before anything is enqueued. */
int nvfp4_moe_plan_w13_swiglu_with_shared(const int32_t *topk_ids, int32_t M, int32_t topk, int32_t E,
                                          void *plan, size_t plan_bytes, const uint16_t *x,
                                          const nvfp4_weights *w13, int32_t layout, uint16_t *h,
                                          const nvfp4_weights *shared_w13, const uint16_t *gate,
                                          uint16_t *shared_h, float *shared_sigma, void *stream);
int nvfp4_moe_w2_reduce_with_shared(const void *plan, int32_t M, int32_t topk, int32_t E, const uint16_t *h,
                                    const nvfp4_weights *w2, const float *topk_weights, const uint16_t *shared_h,
                                    const nvfp4_weights *shared_w2, const float *shared_sigma, float *shared_y,
                                    uint16_t *out, void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------------------------
 * Dense NVFP4 projection (the "QPN" projection, DFlash2 page, "Purpose" and "TP4-only NVFP4
 * verifier follow-up"):
 *   y[m][n] = fp16_rne( global * sum_k x[m][k] * e2m1*e4m3 ),  FP32 accumulation.
 *   x  fp16 [M][K],  w  groups = 1, rows = N, k = K,  y  fp16 [M][N].
 * Any M works. The streaming kernel is tuned for M <= 32, the pages' admitted range.
 * Requirements: K % 128 == 0 and K <= 32768; N % 16 == 0; x, y, codes 16-byte aligned.
 * --------------------------------------------------------------------------------------------- */
int nvfp4_linear(const uint16_t *x, int32_t M, const nvfp4_weights *w, uint16_t *y, void *stream);

/* ---------------------------------------------------------------------------------------------
 * Channel-FP8 dense projection (the "QPN8" path, DFlash2 page, "Follow-up: exact channel-FP8 QPN8
 * concurrency paths and endpoint evidence"):
 *   y[m][n] = fp16_rne( s[n] * sum_k x[m][k] * e4m3(W[n][k]) ),  FP32 accumulation,
 *   x fp16 [M][K], w rows = N, k = K, y fp16 [M][N].
 * The E4M3 bytes convert to fp16 exactly; the channel scale multiplies the FP32 sum (the pages
 * apply it before the MMA). The reduction order is the library's, so a batch is bitwise equal to
 * single-row calls.
 * Requirements: K % 128 == 0 and K <= 16384; N % 16 == 0; x, y, codes 16-byte aligned.
 * --------------------------------------------------------------------------------------------- */
int nvfp4_linear_fp8(const uint16_t *x, int32_t M, const fp8_channel_weights *w, uint16_t *y, void *stream);

/* ---------------------------------------------------------------------------------------------
 * Gated form of the dense projection: the packed gate/up projection of a dense NVFP4 MLP with
 * SwiGLU fused (DFlash2 page, "TP4-only NVFP4 verifier follow-up": the gate/up and down
 * projections of the packed MLP weights; the down projection is nvfp4_linear on h).
 *   x    fp16 [M][K]
 *   w13  groups = 1, rows = 2I, k = K; layout 0: gate rows [0, I), up rows [I, 2I);
 *        layout 1: row 2i is gate i, row 2i+1 is up i
 *   h    fp16 [M][I]
 *   g = global * sum_k x[m,k] * e2m1*e4m3 (gate row i),  u = likewise (up row i),
 *   h[m][i] = fp16_rne( silu(g) * u ),  silu(g) = g / (1 + exp(-g)),  all FP32.
 * The arithmetic is that of nvfp4_moe_w13_swiglu, so h equals a one-expert MoE's W13 bitwise.
 * Requirements: K % 128 == 0 and K <= 16384; I % 16 == 0; x, h, codes 16-byte aligned.
 * --------------------------------------------------------------------------------------------- */
int nvfp4_linear_swiglu(const uint16_t *x, int32_t M, const nvfp4_weights *w13, int32_t layout, uint16_t *h,
                        void *stream);

/* ---------------------------------------------------------------------------------------------
 * Split-K forms of nvfp4_linear and nvfp4_linear_swiglu (same page and sections: the split-K /
 * FP32 reduction order the verifier keeps). Results are bitwise those of the one-launch calls: the
 * same 512-element chunk products, added in the same chunk order, the same epilogue. The
 * reduction is split across blocks instead of inside one, so each CU reads one chunk of x instead
 * of all of it, which pays once M grows (x is read by every block of the one-launch kernel).
 * Two launches: per-chunk FP32 partial products into ws, then their ordered sum.
 *   ws     device memory of at least nvfp4_linear_ws_bytes(M, rows, k) bytes (rows = N, or 2I for
 *          the gated form), 16-byte aligned, owned by the caller; its contents on entry do not
 *          matter and are overwritten (num_chunks(K) * M * rows FP32 values, num_chunks(K) =
 *          ceil(K / 512)). Calls that share a ws must not run concurrently.
 * Arguments, requirements and the other errors are those of nvfp4_linear / nvfp4_linear_swiglu;
 * in addition NVFP4_ERR_NULL for ws == NULL, NVFP4_ERR_ALIGN for a misaligned ws and
 * NVFP4_ERR_WORKSPACE for ws_bytes below the size above, all before anything is enqueued.
 * nvfp4_linear_ws_bytes returns 0 for M < 0, N < 1 or K < 1.
 * --------------------------------------------------------------------------------------------- */
size_t nvfp4_linear_ws_bytes(int32_t M, int32_t N, int32_t K);
int nvfp4_linear_ws(const uint16_t *x, int32_t M, const nvfp4_weights *w, uint16_t *y, void *ws, size_t ws_bytes,
                    void *stream);
int nvfp4_linear_swiglu_ws(const uint16_t *x, int32_t M, const nvfp4_weights *w13, int32_t layout, uint16_t *h,
                           void *ws, size_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4MOE_H */
