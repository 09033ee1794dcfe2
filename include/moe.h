/*
 * moe.h - C ABI of one GPU's share of an expert-parallel Mixture-of-Experts
 * layer on AMD Instinct MI355X (gfx950).
 *
 * The layer (sources named by page title and section):
 *   route     "Mixture-of-experts serving" (learn-kernels), paragraph 1:
 *             sigmoid affinity per expert plus a per-expert bias that only
 *             steers selection; paragraph 4: group-limited routing.
 *             "7.13 Serving Mixture-of-Experts" (llm-stack-book), section
 *             "Expert Parallelism Mechanics", the moe_ep_layer listing:
 *             softmax, top-k, renormalise the chosen k.
 *   dispatch  same chapter, mechanics step 2 (rows of one expert made
 *             contiguous), and "One-Sided Expert-Parallel All-to-All for
 *             Mixture-of-Experts Inference over NVLink" (abstract): each
 *             token is pushed without a metadata exchange into expert-grouped
 *             buffers that the grouped GEMMs read in place.  Here a token
 *             reserves its slot with a per-expert atomic counter.
 *             "DeepEP" section, trick 1: activations quantised to E4M3.
 *   expert    mechanics step 3: one grouped GEMM over all local experts;
 *   ffn       the experts are SwiGLU FFNs, plus the always-on shared expert
 *             ("Hot-Expert Skew" section, "Shared experts as a relief
 *             valve"; learn-kernels paragraph 1).
 *   combine   mechanics step 4 and the moe_ep_layer listing: weighted sum of
 *             each token's k expert outputs, plus the shared expert's output
 *             (DeepEP decode sketch: combine(...) + shared_out).
 *
 * Conventions shared by every entry point
 *   - Every pointer argument is device memory owned by the caller, except
 *     the moe_config / moe_weights structs themselves, which are host memory
 *     read during the call only.  The library never allocates, frees or
 *     synchronises; all work is enqueued on `stream` (a hipStream_t; NULL is
 *     the default stream) and is asynchronous.
 *   - Arguments are checked before anything is launched; a failed check
 *     returns its status and launches nothing.  A failed launch returns
 *     MOE_ERR_HIP.  There is no device-side error reporting.
 *   - T = 0 is valid and launches nothing.
 *   - Row-major layouts throughout; "K-contiguous" means the reduction index
 *     is the fastest-varying one.  Device pointers must be 16-byte aligned.
 *   - Element types: MOE_F32 = IEEE binary32, MOE_BF16 = bfloat16 bit
 *     patterns (uint16), MOE_FP8_E4M3 = OCP E4M3FN bytes (max 448, no inf).
 *   - Apart from the scratch of moe_layer_static, the library holds no
 *     mutable global state: calls on different streams with different
 *     buffers may run concurrently.
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
  MOE_ERR_INVALID_ARG = 1,         /* null/misaligned pointer, bad size or config */
  MOE_ERR_UNSUPPORTED = 2,         /* valid config outside what the kernels cover */
  MOE_ERR_WORKSPACE_TOO_SMALL = 3, /* ws_bytes below the matching *_workspace_size */
  MOE_ERR_HIP = 4,                 /* a HIP launch failed */
  MOE_ERR_SCRATCH_LIMIT = 5        /* moe_layer_static: the call needs more than its static scratch */
} moe_status;

typedef enum { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 } moe_score_fn;

typedef enum {
  MOE_WEIGHT_NORM_SUM = 0,        /* w_j = s_j / sum_i s_i over the chosen k      */
  MOE_WEIGHT_SOFTMAX_SELECTED = 1 /* w_j = exp(s_j) / sum_i exp(s_i) over the k   */
} moe_weight_fn;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3 = 2 } moe_dtype;

/*
 * Layer shape and routing rule.
 *   num_experts E (1..1024), top_k k (1..64, k <= topk_group * E / n_group),
 *   d_model d, d_ff F (routed experts), num_shared (0 or 1), d_ff_shared Fs.
 *   n_group G (1..64, divides E), topk_group kg (1..G):
 *     experts form G contiguous groups of E/G; a group's score is the sum of
 *     its two largest selection keys (its only key when E/G = 1); the kg best
 *     groups are kept and the top k are chosen among their experts.  G = 1
 *     is plain top-k.
 *   score_fn: SIGMOID -> s_e = sigmoid(logit_e), key_e = s_e + bias_e (fp32);
 *             SOFTMAX -> s = softmax(logits), key_e = logit_e (same order).
 *   weight_fn: how the k weights are formed from the unbiased s of the chosen
 *             experts; then every weight is multiplied by routed_scale.
 *   Ties: lower group index, then lower expert index wins.  NaN keys count as
 *   -inf.  topk_idx lists the k experts by descending key.
 *   act_dtype (x and y): MOE_F32 or MOE_BF16.
 *   weight_dtype: MOE_F32 (with act F32), MOE_BF16 (with act BF16) or
 *   MOE_FP8_E4M3 (with act BF16: activations are quantised to E4M3 per
 *   token per 128 columns inside the layer; weights carry 128x128 block
 *   scales).
 *   Size rules: d, F, Fs multiples of 64 (F32), 128 (BF16) or 256 (FP8).
 *   masked_layout: 0 = compact dispatch layout (expert e owns rows
 *             [expert_offset[e], expert_offset[e+1]) of T*k rows, offsets
 *             from a scan of the counters); 1 = masked layout (expert e owns
 *             rows [e*T, e*T + expert_count[e]) of E*T rows: a token's row
 *             follows from its ticket alone, so the router can write it,
 *             with no scan and no dispatch launch).  Same results, more
 *             memory: every per-row buffer has E*T rows instead of T*k.
 */
typedef struct {
  int32_t num_experts;
  int32_t top_k;
  int32_t d_model;
  int32_t d_ff;
  int32_t num_shared;
  int32_t d_ff_shared;
  int32_t n_group;
  int32_t topk_group;
  int32_t score_fn;  /* moe_score_fn  */
  int32_t weight_fn; /* moe_weight_fn */
  float routed_scale;
  int32_t act_dtype;    /* moe_dtype */
  int32_t weight_dtype; /* moe_dtype */
  int32_t masked_layout; /* 0 compact, 1 masked */
} moe_config;

/*
 * Expert weights (device memory, element type weight_dtype, K-contiguous):
 *   w13  [E][2F][d]  rows [0, F) are the gate projection, rows [F, 2F) the up
 *                    projection of each expert
 *   w2   [E][d][F]   down projection
 *   ws13 [2Fs][d], ws2 [d][Fs]  shared expert (NULL when num_shared == 0)
 * FP8 only: fp32 scales per 128 x 128 block of each matrix,
 *   w13_scale [E][2F/128][d/128], w2_scale [E][d/128][F/128],
 *   ws13_scale [2Fs/128][d/128], ws2_scale [d/128][Fs/128];
 *   the weight is code * scale.  Ignored (may be NULL) otherwise.
 */
typedef struct {
  const void* w13;
  const void* w2;
  const void* ws13;
  const void* ws2;
  const float* w13_scale;
  const float* w2_scale;
  const float* ws13_scale;
  const float* ws2_scale;
} moe_weights;

/* Row count of the dispatch buffer for T tokens: the routed rows (T*k in
 * the compact layout, E*T in the masked one), plus T rows holding the
 * quantised tokens for the shared expert when weight_dtype is FP8 and
 * num_shared is 1 (in the bf16 and f32 paths the shared expert reads x
 * directly).  The routed row count also sizes expert_out and row_of's
 * values. */
int64_t moe_dispatch_rows(const moe_config* cfg, int32_t T);

/* Bytes of device workspace moe_expert_ffn needs for up to max_tokens tokens
 * (0 on an invalid config or max_tokens < 0). */
size_t moe_ffn_workspace_size(const moe_config* cfg, int32_t max_tokens);

/* Bytes of device workspace moe_layer needs for up to max_tokens tokens
 * (0 on an invalid config or max_tokens < 0).  The caller zero-fills the
 * workspace once after allocating it; the layer leaves its counters at zero
 * when it returns, so the same workspace serves every later call with the
 * same config (or one with no more experts: the counters are the first E
 * words).  After a call that returned anything but MOE_OK the counters may
 * be left non-zero: zero-fill the workspace again before the next call.  (The kernels bound
 * every row they write or read by the buffers' sizes, so a stale workspace
 * gives wrong results, never an access outside the buffers.) */
size_t moe_workspace_size(const moe_config* cfg, int32_t max_tokens);

/*
 * moe_route: scores, group-limited top-k, gate weights and slot tickets.
 *   logits       [T][E] fp32
 *   bias         [E] fp32, or NULL for no bias (used by SIGMOID only)
 *   topk_idx     [T][k] int32 out: chosen experts, descending key
 *   topk_w       [T][k] fp32 out: gate weights (sum = routed_scale)
 *   expert_count [E] int32 in/out: MUST be zero on entry; on exit holds the
 *                number of (token, slot) pairs routed to each expert (moe_combine
 *                zeroes it again; after a failed call the caller must)
 *   ticket       [T][k] int32 out: the token's slot within its expert's rows,
 *                taken with an atomic add on expert_count; tickets of one
 *                expert are a permutation of 0..count-1 in an unspecified
 *                order
 */
moe_status moe_route(const moe_config* cfg, int32_t T, const float* logits, const float* bias,
                     int32_t* topk_idx, float* topk_w, int32_t* expert_count, int32_t* ticket,
                     void* stream);

/*
 * moe_dispatch: one-sided write of every token into its experts' rows.
 *   x             [T][d] act_dtype
 *   topk_idx, expert_count, ticket: as left by moe_route
 *   recv          [moe_dispatch_rows][d] out: act_dtype, or E4M3 bytes when
 *                 weight_dtype is FP8.  Compact layout: expert e owns rows
 *                 [expert_offset[e], expert_offset[e+1]); token t's slot j
 *                 lands in row expert_offset[topk_idx[t][j]] + ticket[t][j].
 *                 Masked layout: row topk_idx[t][j] * T + ticket[t][j].
 *                 FP8 + shared expert: the row after the routed rows, plus
 *                 t, holds token t.
 *   recv_scale    [moe_dispatch_rows][d/128] fp32 out (FP8 only, else NULL):
 *                 per-row, per-128-column scale; code = E4M3(x / scale) with
 *                 scale = amax / 448 (1 when amax = 0), nearest-even, saturating
 *   expert_offset [E+1] int32 out: exclusive prefix sum of expert_count
 *                 (compact layout; not written, and may be NULL, in the
 *                 masked layout)
 *   row_of        [T][k] int32 out: the row of token t's slot j
 */
moe_status moe_dispatch(const moe_config* cfg, int32_t T, const void* x, const int32_t* topk_idx,
                        const int32_t* expert_count, const int32_t* ticket, void* recv,
                        float* recv_scale, int32_t* expert_offset, int32_t* row_of, void* stream);

/*
 * moe_route_dispatch: moe_route and moe_dispatch in one launch, for the
 * masked layout (masked_layout must be 1; MOE_ERR_INVALID_ARG otherwise).
 * "One-Sided Expert-Parallel All-to-All" (abstract): a token reserves its
 * slot with an atomic add on the expert's counter and is written straight
 * into that slot; with the masked layout the slot's row is known as soon as
 * the ticket is, so the routing wave writes the token itself.
 *   logits, bias, topk_idx, topk_w, expert_count: as for moe_route
 *   ticket        [T][k] int32 out, or NULL when the caller does not need it
 *   x, recv, recv_scale, row_of: as for moe_dispatch (masked layout)
 * Results equal moe_route followed by moe_dispatch.
 */
moe_status moe_route_dispatch(const moe_config* cfg, int32_t T, const float* logits, const float* bias,
                              const void* x, int32_t* topk_idx, float* topk_w, int32_t* expert_count,
                              int32_t* ticket, void* recv, float* recv_scale, int32_t* row_of,
                              void* stream);

/*
 * moe_expert_ffn: grouped SwiGLU experts over the dispatch buffer, read in
 * place, and the shared expert over x.  Experts with no rows read none of
 * their weights.
 *   recv, recv_scale, expert_offset: as left by moe_dispatch.  In the
 *                masked layout pass expert_count (as left by moe_route or
 *                moe_route_dispatch) in place of expert_offset: expert e's
 *                rows are [e*T, e*T + expert_count[e]).
 *   w            expert weights (host struct of device pointers)
 *   x            [T][d] act_dtype (shared expert input; may be NULL when
 *                num_shared == 0)
 *   expert_out   [T*k][d] fp32 out: row r = W2 (silu(Wg a) * (Wu a)) for the
 *                dispatch row a = recv[r]
 *   shared_out   [T][d] fp32 out (NULL when num_shared == 0)
 *   ws, ws_bytes device workspace of at least moe_ffn_workspace_size(cfg, T)
 *                bytes (holds the SwiGLU activations between the two GEMMs)
 */
moe_status moe_expert_ffn(const moe_config* cfg, int32_t T, const void* recv,
                          const float* recv_scale, const int32_t* expert_offset,
                          const moe_weights* w, const void* x, float* expert_out,
                          float* shared_out, void* ws, size_t ws_bytes, void* stream);

/*
 * The two halves of moe_expert_ffn, for callers that schedule them apart
 * (moe_expert_ffn is exactly moe_ffn_gate_up followed by moe_ffn_down on the
 * same workspace).
 *   moe_ffn_gate_up: h = silu(Wg a) * (Wu a) for every dispatch row a and,
 *     with a shared expert, for every token of x; h stays in ws (at least
 *     moe_ffn_workspace_size(cfg, T) bytes; its layout is private).
 *   moe_ffn_down: expert_out[r] = W2 h[r], shared_out[t] = Ws2 hs[t], reading
 *     the h that moe_ffn_gate_up left in ws for the same T and routing.
 */
moe_status moe_ffn_gate_up(const moe_config* cfg, int32_t T, const void* recv, const float* recv_scale,
                           const int32_t* expert_offset, const moe_weights* w, const void* x, void* ws,
                           size_t ws_bytes, void* stream);
moe_status moe_ffn_down(const moe_config* cfg, int32_t T, const int32_t* expert_offset, const moe_weights* w,
                        const void* ws, size_t ws_bytes, float* expert_out, float* shared_out, void* stream);

/*
 * moe_combine: y[t] = sum_j topk_w[t][j] * expert_out[row_of[t][j]]
 * (accumulated in fp32 in slot order j = 0..k-1) + shared_out[t], rounded to
 * act_dtype.  Also resets expert_count[0..E) to zero for the next call.
 *   shared_out may be NULL (no shared term).  y is [T][d] act_dtype.
 */
moe_status moe_combine(const moe_config* cfg, int32_t T, const float* expert_out,
                       const int32_t* row_of, const float* topk_w, const float* shared_out, void* y,
                       int32_t* expert_count, void* stream);

/*
 * moe_router_logits: the router's scores before the score function,
 * logits[t][e] = sum_c x[t][c] * w_router[e][c], accumulated in fp32
 * ("7.13 Serving Mixture-of-Experts", moe_ep_layer listing: the router is a
 * linear map of the token to one score per expert, followed by the softmax
 * and top-k that moe_route applies).  Its output is moe_route's (and
 * moe_layer's) logits input.
 *   x        [T][d] act_dtype (bf16 for the bf16 and E4M3 layers, fp32 for
 *            the fp32 layer), K-contiguous.
 *   w_router [E][d] act_dtype, K-contiguous (one row per expert).
 *   logits   [T][E] fp32, written.
 * The products are exact in fp32 and are summed in fp32 in a fixed order, so
 * the result is reproducible run to run.  Requires E % 64 == 0
 * (MOE_ERR_UNSUPPORTED otherwise).  Needs no workspace (moe_router_logits_ws,
 * below, takes one to run larger batches faster).
 */
moe_status moe_router_logits(const moe_config* cfg, int32_t T, const void* x, const void* w_router,
                             float* logits, void* stream);

/*
 * moe_router_logits_ws: moe_router_logits with a caller workspace, which lets
 * the product's reduction (the sum over c) be split over workgroups where
 * moe_router_logits would leave most of the GPU idle: bf16 layers with
 * E % 128 == 0, from 256 tokens on when d_model >= 4096, else from 1024.  Each of P parts sums its share of c in fp32
 * into ws, and a second launch adds the P partial sums in part order, so the
 * result is reproducible run to run; it may differ from moe_router_logits'
 * in the last bits (another summation order).  Elsewhere the call is
 * moe_router_logits and ws is not touched.
 *   x, w_router, logits: as for moe_router_logits.
 *   ws, ws_bytes: at least moe_router_workspace_size(cfg, T) bytes, 16-byte
 *   aligned, no initial contents needed (scratch, overwritten); may be NULL
 *   when that size is 0.  MOE_ERR_WORKSPACE_TOO_SMALL when ws_bytes is
 *   smaller, nothing launched.
 */
moe_status moe_router_logits_ws(const moe_config* cfg, int32_t T, const void* x, const void* w_router,
                                float* logits, void* ws, size_t ws_bytes, void* stream);

/* Bytes of workspace moe_router_logits_ws needs for any T <= max_tokens (0:
 * it splits nothing there).  0 for an invalid cfg or max_tokens < 0. */
size_t moe_router_workspace_size(const moe_config* cfg, int32_t max_tokens);

/*
 * moe_layer: route -> dispatch -> expert FFN (+ shared expert) -> combine in
 * one call, every intermediate carved from ws (>= moe_workspace_size(cfg, T)
 * bytes, zero-filled once by the caller).  Launches only; no host sync, so
 * the sequence can be captured in a HIP graph.  With the masked layout the
 * route and dispatch steps are one launch (moe_route_dispatch).
 */
moe_status moe_layer(const moe_config* cfg, int32_t T, const void* x, const float* logits,
                     const float* bias, const moe_weights* w, void* y, void* ws, size_t ws_bytes,
                     void* stream);

/*
 * moe_layer_fused: the whole layer for a handful of tokens in ONE persistent
 * launch ("DeepSeek MoE Serving: Where Expert-Parallel All-to-All Time
 * Goes", section "The batch-scaling curve is the diagnostic": a fused MoE
 * kernel running dispatch, both expert GEMMs and combine in one kernel;
 * "7.13 Serving Mixture-of-Experts", "DeepEP" trick 3: at decode batch sizes
 * the per-layer launch overhead can rival the work).  Optionally it starts
 * from the hidden states and computes the router logits itself (the
 * moe_ep_layer listing's x @ router_w^T).
 *   Exactly one of logits ([T][E] fp32, as for moe_layer) and w_router
 *   ([E][d] bf16, as for moe_router_logits) is non-NULL; with w_router the
 *   logits are computed in the launch, with moe_router_logits' arithmetic.
 *   x, bias, w, y: as for moe_layer.  masked_layout is ignored.
 *   ws, ws_bytes: workspace of at least moe_fused_workspace_size(cfg, T)
 *   bytes, zero-filled once by the caller.  Its first 12 KB hold the grid
 *   barriers' counters and flags, which the launch leaves at zero, so the
 *   same workspace serves every later call; the rest is scratch the launch
 *   writes before it reads.  The int at byte 16 of ws is set to 1 (and never
 *   cleared by the library) when one of the launch's bounded grid-wide waits
 *   gave up (for instance on counters that were not zero): the results of
 *   that call are then invalid.
 *   Supported (else MOE_ERR_UNSUPPORTED, nothing launched): bf16 activations
 *   and weights, 1 <= T <= 16, T*k <= 256, E <= 256, d, d_ff and d_ff_shared
 *   multiples of 128, d <= 16384 when w_router is given (moe_fused_supported
 *   tells).  Routing and weights follow moe_layer exactly; each token's
 *   expert outputs are added in a fixed order (ascending expert, then the
 *   shared expert) with no atomics, so the output is reproducible bit for
 *   bit run to run.
 *   The launch keeps one workgroup on every CU and synchronises them with
 *   grid-wide barriers: it must not share the GPU with another launch that
 *   occupies every CU for long (it waits for CUs, within its bound).
 */
moe_status moe_layer_fused(const moe_config* cfg, int32_t T, const void* x, const float* logits, const void* w_router,
                           const float* bias, const moe_weights* w, void* y, void* ws, size_t ws_bytes,
                           void* stream);
size_t moe_fused_workspace_size(const moe_config* cfg, int32_t max_tokens);
int32_t moe_fused_supported(const moe_config* cfg, int32_t T);

/*
 * moe_layer_static: moe_layer without a workspace argument and without any
 * allocation, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).  The
 * intermediates live in a scratch array inside the library, one copy of
 * moe_layer_static_max_bytes() bytes (64 MiB) per GPU, held until the process
 * ends.  Arguments and results are those of moe_layer.
 *   Returns MOE_ERR_SCRATCH_LIMIT, launching nothing, when the call needs more
 *   than that (moe_workspace_size(cfg, T) > moe_layer_static_max_bytes():
 *   e.g. the DeepSeek-V3-shaped bf16 layer fits up to about 160 tokens in
 *   the compact layout, the Qwen3-30B-A3B-shaped one about 600).
 *   Every call on a GPU shares that GPU's scratch, whatever its config.  The
 *   library keeps the routing counters zero between calls (a fill kernel on a
 *   device's first call, after a call that returned an error, and before a
 *   call whose config has more experts than the previous call's); calls that
 *   overlap on one GPU (other streams or threads) race on the scratch and
 *   must be serialised by the caller.
 */
moe_status moe_layer_static(const moe_config* cfg, int32_t T, const void* x, const float* logits,
                            const float* bias, const moe_weights* w, void* y, void* stream);
size_t moe_layer_static_max_bytes(void);

/* Static, human-readable name of a status code. */
const char* moe_status_string(moe_status status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
