/*
 * moe_ref.h - plain C++ CPU oracle of one GPU's share of an expert-parallel
 * Mixture-of-Experts layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's cpu_baseline leg load this library.  It shares no code, header,
 * table or helper with the GPU library: it is the layer written out as the
 * pages define it, in loops, with every dot product and reduction accumulated
 * in double.
 *
 * Sources (page title, then section):
 *   route    "Mixture-of-experts serving" (learn-kernels), paragraph 1
 *            (sigmoid affinity plus a per-expert bias that only steers
 *            selection) and paragraph 4 (group-limited routing);
 *            "7.13 Serving Mixture-of-Experts" (llm-stack-book), section
 *            "Expert Parallelism Mechanics", moe_ep_layer listing (softmax,
 *            top-k, renormalise the chosen k).
 *   dispatch same section, steps 1-2: every (token, slot) pair goes to its
 *            expert, the rows of one expert contiguous (here in ascending
 *            token order: the canonical layout).
 *   ffn      same section, step 3 (one matmul pair per expert), with SwiGLU
 *            experts; the shared expert on every token ("Hot-Expert Skew",
 *            shared experts; learn-kernels paragraph 1).
 *   combine  same section, step 4 and the listing: the weighted sum of each
 *            token's k expert outputs, plus the shared expert's output
 *            ("DeepEP" section, decode sketch: combine(...) + shared_out).
 *   E4M3     "DeepEP" section, trick 1: activations sent as E4M3; the codec
 *            follows the OCP 8-bit floating point format (bias 7, three
 *            mantissa bits, max 448, S.1111.111 NaN, no infinity).
 *
 * Conventions: every pointer is host memory owned by the caller; outputs are
 * double unless stated.  Functions return 0 on success and -1 on an invalid
 * argument.  nthreads = 0 uses every hardware thread; results do not depend
 * on it (each output element is computed by one thread in a fixed order).
 */
#ifndef MOE_REF_H
#define MOE_REF_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types of x and of the weights */
enum { MOE_REF_F32 = 0, MOE_REF_BF16 = 1, MOE_REF_E4M3 = 2, MOE_REF_F64 = 3 };

typedef struct {
  int32_t num_experts, top_k, d_model, d_ff, num_shared, d_ff_shared, n_group, topk_group;
  int32_t score_fn;   /* 0 softmax over all experts, 1 sigmoid + bias */
  int32_t weight_fn;  /* 0 normalise the chosen k to sum 1, 1 softmax over the chosen k */
  double routed_scale;
  int32_t act_dtype;    /* x: MOE_REF_F32, MOE_REF_BF16 or MOE_REF_F64 */
  int32_t weight_dtype; /* MOE_REF_F32, MOE_REF_BF16, MOE_REF_E4M3 (+ 128x128 block scales) or MOE_REF_F64 */
  int32_t act_quant;    /* 1: quantise the rows entering both GEMMs per 1x128 block to E4M3 (x, and h
                           rounded to fp32), as the E4M3 kernels do; 0: exact activations */
} moe_ref_config;

/* w13 [E][2F][d] (gate rows [0,F), up rows [F,2F)), w2 [E][d][F], ws13 [2Fs][d],
 * ws2 [d][Fs]; E4M3: fp32 scales per 128x128 block, weight = code * scale. */
typedef struct {
  const void* w13;
  const void* w2;
  const void* ws13;
  const void* ws2;
  const float* w13_scale;
  const float* w2_scale;
  const float* ws13_scale;
  const float* ws2_scale;
} moe_ref_weights;

/* Selection keys [T][E] fp32: sigmoid -> fp32(sigmoid(l)) + bias (fp32 add),
 * softmax -> l; NaN -> -inf. */
int moe_ref_keys(const moe_ref_config* c, int32_t T, const float* logits, const float* bias, float* keys);

/* Routing: topk_idx [T][k] by descending key (ties: lower index), weights
 * [T][k] from the unbiased scores, times routed_scale.  Group-limited when
 * n_group > 1: a group's score is the fp32 sum of its two largest keys (its
 * only key when a group holds one expert); the topk_group best groups (ties:
 * lower group) are eligible. */
int moe_ref_route(const moe_ref_config* c, int32_t T, const float* logits, const float* bias,
                  int32_t* topk_idx, double* topk_w);

/* Gate weights of a given selection (as moe_ref_route computes them). */
int moe_ref_gate_weights(const moe_ref_config* c, int32_t T, const float* logits, const int32_t* topk_idx,
                         double* topk_w);

/* Per-token closeness to a tie: the gap between the k-th and (k+1)-th
 * eligible keys, and (grouped routing) between the topk_group-th and next
 * group scores; the smaller one, in double (+inf when no competitor). */
int moe_ref_margins(const moe_ref_config* c, int32_t T, const float* logits, const float* bias, double* gap);

/* Canonical dispatch: counts [E], offsets [E+1], row_of [T][k], token_of_row
 * [T*k]; the rows of expert e are [offsets[e], offsets[e+1]) in ascending
 * token order. */
int moe_ref_dispatch(const moe_ref_config* c, int32_t T, const int32_t* topk_idx, int32_t* counts,
                     int32_t* offsets, int32_t* row_of, int32_t* token_of_row);

/* recv [T*k][d] double: the dispatched rows x[token_of_row[r]]. */
int moe_ref_gather(const moe_ref_config* c, int32_t T, const void* x, const int32_t* token_of_row, double* recv);

/* Grouped SwiGLU experts over recv (rows of expert e at offsets), and the
 * shared expert over x: expert_out [T*k][d], shared_out [T][d] (NULL without
 * a shared expert). */
int moe_ref_expert_ffn(const moe_ref_config* c, int32_t T, const double* recv, const int32_t* offsets,
                       const moe_ref_weights* w, const void* x, double* expert_out, double* shared_out,
                       int32_t nthreads);

/* y[t] = sum_j w[t][j] expert_out[row_of[t][j]] (j in order) + shared_out[t]. */
int moe_ref_combine(const moe_ref_config* c, int32_t T, const double* expert_out, const int32_t* row_of,
                    const double* topk_w, const double* shared_out, double* y);

/* The layer: route, dispatch, expert FFNs, shared expert, combine.  With
 * topk_idx and topk_w non-NULL the given routing is used instead (both in). */
int moe_ref_layer(const moe_ref_config* c, int32_t T, const void* x, const float* logits, const float* bias,
                  const moe_ref_weights* w, const int32_t* topk_idx, const double* topk_w, double* y,
                  int32_t nthreads);

/* Brute-force output of one token: its k experts and the shared expert
 * straight from x and the weights, with no dispatch buffer. */
int moe_ref_dense_token(const moe_ref_config* c, const void* x_row, const int32_t* idx_row, const double* w_row,
                        const moe_ref_weights* w, double* y_row);

/* logits[t][e] = sum_c x[t][c] w_router[e][c] in double (act dtype for both). */
int moe_ref_router_logits(const moe_ref_config* c, int32_t T, const void* x, const void* w_router,
                          double* logits);

/* E4M3 codec: the value of a code; the nearest code of an fp32 value (ties
 * to the even code, saturating at +-448, -0 -> +0, NaN -> 0x7F). */
double moe_ref_e4m3_decode(uint8_t code);
uint8_t moe_ref_e4m3_encode(float v);

/* Per-row, per-128-column quantisation of fp32 rows [n][d]: scale = fp32
 * amax / 448 (1 when amax = 0), code = encode(fp32(x / scale)). */
int moe_ref_quantize_rows(int64_t n, int64_t d, const float* x, uint8_t* codes, float* scales);

#ifdef __cplusplus
}
#endif

#endif /* MOE_REF_H */
