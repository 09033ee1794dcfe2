// C ABI: argument checks, workspace carving and kernel launches.  No host
// synchronisation, no allocation: every call only enqueues work on the
// caller's stream.
#include <math.h>
#include <string.h>

#include "moe_kernels.h"

using namespace moe;

namespace {

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int elem_bytes(int dt) { return dt == MOE_F32 ? 4 : dt == MOE_BF16 ? 2 : 1; }

moe_status check_config(const moe_config* c) {
  if (!c) return MOE_ERR_INVALID_ARG;
  const int E = c->num_experts, k = c->top_k, G = c->n_group, kg = c->topk_group;
  if (E < 1 || E > 1024 || k < 1 || k > 64 || k > E) return MOE_ERR_INVALID_ARG;
  if (c->d_model <= 0 || c->d_ff <= 0) return MOE_ERR_INVALID_ARG;
  if (c->num_shared != 0 && c->num_shared != 1) return MOE_ERR_INVALID_ARG;
  if (c->num_shared == 1 && c->d_ff_shared <= 0) return MOE_ERR_INVALID_ARG;
  if (G < 1 || G > 64 || E % G != 0 || kg < 1 || kg > G) return MOE_ERR_INVALID_ARG;
  if (k > kg * (E / G)) return MOE_ERR_INVALID_ARG;
  if (c->score_fn != MOE_SCORE_SOFTMAX && c->score_fn != MOE_SCORE_SIGMOID) return MOE_ERR_INVALID_ARG;
  if (c->weight_fn != MOE_WEIGHT_NORM_SUM && c->weight_fn != MOE_WEIGHT_SOFTMAX_SELECTED) return MOE_ERR_INVALID_ARG;
  if (!isfinite(c->routed_scale)) return MOE_ERR_INVALID_ARG;
  const int a = c->act_dtype, w = c->weight_dtype;
  if (a < MOE_F32 || a > MOE_FP8_E4M3 || w < MOE_F32 || w > MOE_FP8_E4M3) return MOE_ERR_INVALID_ARG;
  const bool combo = (a == MOE_F32 && w == MOE_F32) || (a == MOE_BF16 && w == MOE_BF16) ||
                     (a == MOE_BF16 && w == MOE_FP8_E4M3);
  if (!combo) return MOE_ERR_UNSUPPORTED;
  const int mult = w == MOE_F32 ? 64 : w == MOE_BF16 ? 128 : 256;
  if (c->d_model % mult || c->d_ff % mult) return MOE_ERR_UNSUPPORTED;
  if (c->num_shared && c->d_ff_shared % mult) return MOE_ERR_UNSUPPORTED;
  if (c->masked_layout != 0 && c->masked_layout != 1) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

bool masked(const moe_config* c) { return c->masked_layout == 1; }

// routed rows of every per-row buffer: T*k (compact) or E*T (masked)
int64_t routed_rows(const moe_config* c, int64_t T) { return masked(c) ? T * c->num_experts : T * c->top_k; }

bool fp8(const moe_config* c) { return c->weight_dtype == MOE_FP8_E4M3; }

// dtype of the dispatch buffer rows and of the SwiGLU activations
int recv_dtype(const moe_config* c) { return fp8(c) ? MOE_FP8_E4M3 : c->act_dtype; }

int64_t dispatch_rows(const moe_config* c, int64_t T) {
  return routed_rows(c, T) + ((fp8(c) && c->num_shared) ? T : 0);
}

// row indices are int32 (row_of)
bool rows_fit(const moe_config* c, int64_t T) { return dispatch_rows(c, T) <= 0x7FFFFFFF; }

struct FfnLayout {
  size_t h, h_scale, hs, hs_scale, total;
};

FfnLayout ffn_layout(const moe_config* c, int64_t T) {
  FfnLayout L{};
  const size_t eb = elem_bytes(recv_dtype(c));
  const size_t rows = (size_t)routed_rows(c, T);
  size_t o = 0;
  L.h = o;
  o = align256(o + rows * c->d_ff * eb);
  L.h_scale = o;
  if (fp8(c)) o = align256(o + rows * (c->d_ff / 128) * sizeof(float));
  L.hs = o;
  if (c->num_shared) o = align256(o + (size_t)T * c->d_ff_shared * eb);
  L.hs_scale = o;
  if (c->num_shared && fp8(c)) o = align256(o + (size_t)T * (c->d_ff_shared / 128) * sizeof(float));
  L.total = o;
  return L;
}

struct LayerLayout {
  size_t count, idx, w, ticket, row_of, offset, recv, recv_scale, eout, sout, ffn, total;
};

// expert_count sits at offset 0 for every T, so the zero invariant that
// moe_combine restores carries over between calls of any size.
LayerLayout layer_layout(const moe_config* c, int64_t T) {
  LayerLayout L{};
  const size_t tk = (size_t)T * c->top_k, d = c->d_model;
  const size_t rows = (size_t)dispatch_rows(c, T);
  size_t o = 0;
  L.count = o;  o = align256(o + (size_t)c->num_experts * 4);
  L.idx = o;    o = align256(o + tk * 4);
  L.w = o;      o = align256(o + tk * 4);
  L.ticket = o; o = align256(o + tk * 4);
  L.row_of = o; o = align256(o + tk * 4);
  L.offset = o; o = align256(o + (size_t)(c->num_experts + 1) * 4);
  L.recv = o;   o = align256(o + rows * d * elem_bytes(recv_dtype(c)));
  L.recv_scale = o;
  if (fp8(c)) o = align256(o + rows * (d / 128) * sizeof(float));
  L.eout = o;   o = align256(o + (size_t)routed_rows(c, T) * d * sizeof(float));
  L.sout = o;
  if (c->num_shared) o = align256(o + (size_t)T * d * sizeof(float));
  L.ffn = o;    o = align256(o + ffn_layout(c, T).total);
  L.total = o;
  return L;
}

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

template <typename... P>
bool all_aligned(P... ps) { return (aligned16(ps) && ...); }

RouteParams route_params(const moe_config* c, int32_t T, const float* logits, const float* bias, int32_t* idx,
                         float* w, int32_t* count, int32_t* ticket) {
  RouteParams p{};
  p.T = T; p.E = c->num_experts; p.k = c->top_k; p.n_group = c->n_group; p.topk_group = c->topk_group;
  p.score_fn = c->score_fn; p.weight_fn = c->weight_fn; p.routed_scale = c->routed_scale;
  p.logits = logits; p.bias = bias; p.topk_idx = idx; p.topk_w = w; p.expert_count = count; p.ticket = ticket;
  return p;
}

// the router also writes every token into its masked-layout rows
void fuse_dispatch(RouteParams& p, const moe_config* c, const void* x, void* recv, float* recv_scale,
                   int32_t* row_of) {
  p.fuse = 1; p.d = c->d_model; p.act_dtype = c->act_dtype;
  p.quant = fp8(c) ? 1 : 0;
  p.shared_rows = (fp8(c) && c->num_shared) ? 1 : 0;
  p.x = x; p.recv = recv; p.recv_scale = recv_scale; p.row_of = row_of;
}

moe_status route_impl(const moe_config* c, int32_t T, const float* logits, const float* bias, int32_t* idx,
                      float* w, int32_t* count, int32_t* ticket, hipStream_t s) {
  return hip_status(launch_route(route_params(c, T, logits, bias, idx, w, count, ticket), s));
}

moe_status dispatch_impl(const moe_config* c, int32_t T, const void* x, const int32_t* idx, const int32_t* count,
                         const int32_t* ticket, void* recv, float* recv_scale, int32_t* offset, int32_t* row_of,
                         hipStream_t s) {
  DispatchParams p{};
  p.T = T; p.E = c->num_experts; p.k = c->top_k; p.d = c->d_model; p.act_dtype = c->act_dtype;
  p.quant = fp8(c) ? 1 : 0;
  p.shared_rows = (fp8(c) && c->num_shared) ? 1 : 0;
  p.masked = masked(c) ? 1 : 0;
  p.routed_rows = (int)routed_rows(c, T);
  p.x = x; p.topk_idx = idx; p.expert_count = count; p.ticket = ticket; p.recv = recv; p.recv_scale = recv_scale;
  p.expert_offset = offset; p.row_of = row_of;
  return hip_status(launch_dispatch(p, s));
}

FfnParams gate_up_params(const moe_config* c, int32_t T, const void* recv, const float* recv_scale,
                         const int32_t* offset, const moe_weights* W, const void* x, void* ws) {
  const FfnLayout L = ffn_layout(c, T);
  uint8_t* base = static_cast<uint8_t*>(ws);
  const bool q = fp8(c);
  const int d = c->d_model, F = c->d_ff, Fs = c->d_ff_shared, ns = c->num_shared;
  FfnParams a{};
  a.E = c->num_experts; a.T = T; a.expert_offset = offset; a.masked = masked(c) ? 1 : 0; a.n_shared = ns;
  a.tiles_r = F / 16; a.tiles_s = ns ? Fs / 16 : 0;
  a.act = static_cast<const uint8_t*>(recv); a.act_scale = recv_scale;
  a.w = static_cast<const uint8_t*>(W->w13); a.w_scale = W->w13_scale;
  a.K_r = d; a.NW_r = 2 * F; a.Nout_r = F;
  a.out = base + L.h; a.out_scale = q ? reinterpret_cast<float*>(base + L.h_scale) : nullptr;
  if (ns) {
    if (q) {
      a.s_act = static_cast<const uint8_t*>(recv) + (size_t)routed_rows(c, T) * d;
      a.s_act_scale = recv_scale + (size_t)routed_rows(c, T) * (d / 128);
    } else {
      a.s_act = static_cast<const uint8_t*>(x);
    }
    a.s_w = static_cast<const uint8_t*>(W->ws13); a.s_w_scale = W->ws13_scale;
    a.K_s = d; a.NW_s = 2 * Fs; a.Nout_s = Fs;
    a.s_out = base + L.hs; a.s_out_scale = q ? reinterpret_cast<float*>(base + L.hs_scale) : nullptr;
  }
  return a;
}

FfnParams down_params(const moe_config* c, int32_t T, const int32_t* offset, const moe_weights* W,
                      const void* ws, float* eout, float* sout) {
  const FfnLayout L = ffn_layout(c, T);
  const uint8_t* base = static_cast<const uint8_t*>(ws);
  const bool q = fp8(c);
  const int d = c->d_model, F = c->d_ff, Fs = c->d_ff_shared, ns = c->num_shared;
  FfnParams b{};
  b.E = c->num_experts; b.T = T; b.expert_offset = offset; b.masked = masked(c) ? 1 : 0; b.n_shared = ns;
  b.tiles_r = d / 16; b.tiles_s = ns ? d / 16 : 0;
  b.act = base + L.h; b.act_scale = q ? reinterpret_cast<const float*>(base + L.h_scale) : nullptr;
  b.w = static_cast<const uint8_t*>(W->w2); b.w_scale = W->w2_scale;
  b.K_r = F; b.NW_r = d; b.Nout_r = d;
  b.out = eout;
  if (ns) {
    b.s_act = base + L.hs; b.s_act_scale = q ? reinterpret_cast<const float*>(base + L.hs_scale) : nullptr;
    b.s_w = static_cast<const uint8_t*>(W->ws2); b.s_w_scale = W->ws2_scale;
    b.K_s = Fs; b.NW_s = d; b.Nout_s = d;
    b.s_out = sout;
  }
  return b;
}

int max_groups_of(const moe_config* c, int32_t T) {
  const int64_t tk = (int64_t)T * c->top_k;
  return (int)(tk < c->num_experts ? tk : c->num_experts);
}

// no expert takes a token twice and the shared expert takes all T, so no
// group has more than T rows
// Batches with enough rows per expert take the LDS-tiled bf16 kernel, which
// streams each weight tile once per 128 token rows; smaller ones take the
// weight-streaming kernel, which streams it once per 16-row chunk.  The
// crossover falls with the row length (the tiled kernel's per-item cost is
// spread over more K-steps), measured as whole-layer A/B runs:
//   d_model 7168 (256 experts, top 8): 4 rows per expert (128 tokens)
//     streaming 2809 / tiled 2850 us; 5 rows 2973 / 2861; 6 rows 3232 / 2919;
//     12 rows 4532 / 3157; 24 rows 7289 / 3528;
//   d_model 2048 (128 experts, top 8): 8 rows 231 / 250 us; 10 rows 236 /
//     250; 12 rows 256 / 256; 14 rows 272 / 257; 16 rows 308 / 261.
bool use_tiled(const moe_config* c, int32_t T) {
  if (c->weight_dtype != MOE_BF16) return false;
  const int rows_per_expert = c->d_model >= 6144 ? 5 : c->d_model >= 3072 ? 8 : 12;
  return (int64_t)T * c->top_k >= (int64_t)rows_per_expert * c->num_experts;
}

// bound on the 128-row token tiles over all routed groups
long long tiled_token_tiles(const moe_config* c, int32_t T) {
  const long long tk = (long long)T * c->top_k;
  return (tk + 127) / 128 + max_groups_of(c, T);
}

moe_status gate_up_impl(const moe_config* c, int32_t T, const void* recv, const float* recv_scale,
                        const int32_t* offset, const moe_weights* W, const void* x, void* ws, hipStream_t s) {
  const FfnParams a = gate_up_params(c, T, recv, recv_scale, offset, W, x, ws);
  if (use_tiled(c, T))
    return hip_status(launch_gemm_tiled(a, true, tiled_token_tiles(c, T), s));
  return hip_status(launch_ffn(a, c->weight_dtype, true, (long long)T * c->top_k, max_groups_of(c, T), s));
}

moe_status down_impl(const moe_config* c, int32_t T, const int32_t* offset, const moe_weights* W, const void* ws,
                     float* eout, float* sout, hipStream_t s) {
  const FfnParams b = down_params(c, T, offset, W, ws, eout, sout);
  if (use_tiled(c, T))
    return hip_status(launch_gemm_tiled(b, false, tiled_token_tiles(c, T), s));
  return hip_status(launch_ffn(b, c->weight_dtype, false, (long long)T * c->top_k, max_groups_of(c, T), s));
}

moe_status ffn_impl(const moe_config* c, int32_t T, const void* recv, const float* recv_scale,
                    const int32_t* offset, const moe_weights* W, const void* x, float* eout, float* sout,
                    void* ws, hipStream_t s) {
  moe_status st = gate_up_impl(c, T, recv, recv_scale, offset, W, x, ws, s);
  if (st != MOE_OK) return st;
  return down_impl(c, T, offset, W, ws, eout, sout, s);
}

moe_status combine_impl(const moe_config* c, int32_t T, const float* eout, const int32_t* row_of,
                        const float* w, const float* sout, void* y, int32_t* count, hipStream_t s) {
  CombineParams p{};
  p.T = T; p.E = c->num_experts; p.k = c->top_k; p.d = c->d_model; p.act_dtype = c->act_dtype;
  p.routed_rows = (int)routed_rows(c, T);
  p.expert_out = eout; p.row_of = row_of; p.topk_w = w; p.shared_out = sout; p.y = y; p.expert_count = count;
  return hip_status(launch_combine(p, s));
}

// ---- the fused decode layer (fused.hip)

constexpr int kFusedSpinLimit = 1 << 18;  // polls per grid barrier before giving up (about 0.1-0.3 s)

struct FusedLayout {
  size_t sync, logits, h, total;
};

moe_config compact_of(const moe_config* c) {
  moe_config cc = *c;
  cc.masked_layout = 0;
  return cc;
}

// The words that are zero between calls first (an exit count, the error word,
// then two 4 KB barrier blocks), so that the zero invariant carries over
// between calls of any size; then the router's logits [T][E] f32 and h:
// [T*k][F] bf16 (routed slots), [T][Fs] bf16 (shared expert)
constexpr size_t kFusedSyncBytes = 3 * kFusedBarWords * sizeof(int);

FusedLayout fused_layout(const moe_config* c, int64_t T) {
  FusedLayout L{};
  size_t o = 0;
  L.sync = o;   o = align256(o + kFusedSyncBytes);
  L.logits = o; o = align256(o + (size_t)T * c->num_experts * sizeof(float));
  L.h = o;      o = align256(o + (size_t)T * c->top_k * c->d_ff * 2 + (c->num_shared ? (size_t)T * c->d_ff_shared * 2 : 0));
  L.total = o;
  return L;
}

bool fused_ok(const moe_config* c, int32_t T) {
  if (c->act_dtype != MOE_BF16 || c->weight_dtype != MOE_BF16) return false;
  return fused_shape_ok(T, c->top_k, c->num_experts, c->d_model, c->d_ff, c->num_shared ? c->d_ff_shared : 0);
}

moe_status check_weights(const moe_config* c, const moe_weights* W) {
  if (!W || !W->w13 || !W->w2) return MOE_ERR_INVALID_ARG;
  if (!all_aligned(W->w13, W->w2)) return MOE_ERR_INVALID_ARG;
  if (c->num_shared && (!W->ws13 || !W->ws2 || !all_aligned(W->ws13, W->ws2))) return MOE_ERR_INVALID_ARG;
  if (fp8(c)) {
    if (!W->w13_scale || !W->w2_scale) return MOE_ERR_INVALID_ARG;
    if (c->num_shared && (!W->ws13_scale || !W->ws2_scale)) return MOE_ERR_INVALID_ARG;
  }
  return MOE_OK;
}

}  // namespace

extern "C" {

int64_t moe_dispatch_rows(const moe_config* cfg, int32_t T) {
  if (check_config(cfg) != MOE_OK || T < 0) return -1;
  return dispatch_rows(cfg, T);
}

size_t moe_ffn_workspace_size(const moe_config* cfg, int32_t max_tokens) {
  if (check_config(cfg) != MOE_OK || max_tokens < 0) return 0;
  return ffn_layout(cfg, max_tokens).total;
}

size_t moe_workspace_size(const moe_config* cfg, int32_t max_tokens) {
  if (check_config(cfg) != MOE_OK || max_tokens < 0) return 0;
  return layer_layout(cfg, max_tokens).total;
}

moe_status moe_route(const moe_config* cfg, int32_t T, const float* logits, const float* bias, int32_t* topk_idx,
                     float* topk_w, int32_t* expert_count, int32_t* ticket, void* stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (T < 0 || !rows_fit(cfg, T)) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_idx || !topk_w || !expert_count || !ticket) return MOE_ERR_INVALID_ARG;
  if (!all_aligned(logits, topk_idx, topk_w, expert_count, ticket) || (bias && !aligned16(bias)))
    return MOE_ERR_INVALID_ARG;
  return route_impl(cfg, T, logits, bias, topk_idx, topk_w, expert_count, ticket, (hipStream_t)stream);
}

moe_status moe_dispatch(const moe_config* cfg, int32_t T, const void* x, const int32_t* topk_idx,
                        const int32_t* expert_count, const int32_t* ticket, void* recv, float* recv_scale,
                        int32_t* expert_offset, int32_t* row_of, void* stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (T < 0 || !rows_fit(cfg, T)) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!x || !topk_idx || !expert_count || !ticket || !recv || !row_of) return MOE_ERR_INVALID_ARG;
  if (!masked(cfg) && !expert_offset) return MOE_ERR_INVALID_ARG;
  if (fp8(cfg) && !recv_scale) return MOE_ERR_INVALID_ARG;
  if (!all_aligned(x, topk_idx, expert_count, ticket, recv, row_of) || (expert_offset && !aligned16(expert_offset)))
    return MOE_ERR_INVALID_ARG;
  if (recv_scale && !aligned16(recv_scale)) return MOE_ERR_INVALID_ARG;
  return dispatch_impl(cfg, T, x, topk_idx, expert_count, ticket, recv, recv_scale, expert_offset, row_of,
                       (hipStream_t)stream);
}

moe_status moe_route_dispatch(const moe_config* cfg, int32_t T, const float* logits, const float* bias,
                              const void* x, int32_t* topk_idx, float* topk_w, int32_t* expert_count,
                              int32_t* ticket, void* recv, float* recv_scale, int32_t* row_of, void* stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!masked(cfg)) return MOE_ERR_INVALID_ARG;
  if (T < 0 || !rows_fit(cfg, T)) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!logits || !x || !topk_idx || !topk_w || !expert_count || !recv || !row_of) return MOE_ERR_INVALID_ARG;
  if (fp8(cfg) && !recv_scale) return MOE_ERR_INVALID_ARG;
  if (!all_aligned(logits, x, topk_idx, topk_w, expert_count, recv, row_of) || (bias && !aligned16(bias)) ||
      (ticket && !aligned16(ticket)) || (recv_scale && !aligned16(recv_scale)))
    return MOE_ERR_INVALID_ARG;
  RouteParams p = route_params(cfg, T, logits, bias, topk_idx, topk_w, expert_count, ticket);
  fuse_dispatch(p, cfg, x, recv, fp8(cfg) ? recv_scale : nullptr, row_of);
  return hip_status(launch_route(p, (hipStream_t)stream));
}

moe_status moe_expert_ffn(const moe_config* cfg, int32_t T, const void* recv, const float* recv_scale,
                          const int32_t* expert_offset, const moe_weights* w, const void* x, float* expert_out,
                          float* shared_out, void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (T < 0 || !rows_fit(cfg, T)) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if ((st = check_weights(cfg, w)) != MOE_OK) return st;
  if (!recv || !expert_offset || !expert_out || !ws) return MOE_ERR_INVALID_ARG;
  if (fp8(cfg) && !recv_scale) return MOE_ERR_INVALID_ARG;
  if (cfg->num_shared && (!shared_out || (!fp8(cfg) && !x))) return MOE_ERR_INVALID_ARG;
  if (!all_aligned(recv, expert_offset, expert_out, ws)) return MOE_ERR_INVALID_ARG;
  if ((recv_scale && !aligned16(recv_scale)) || (x && !aligned16(x)) || (shared_out && !aligned16(shared_out)))
    return MOE_ERR_INVALID_ARG;
  if (ws_bytes < ffn_layout(cfg, T).total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  return ffn_impl(cfg, T, recv, recv_scale, expert_offset, w, x, expert_out, shared_out, ws, (hipStream_t)stream);
}

moe_status moe_ffn_gate_up(const moe_config* cfg, int32_t T, const void* recv, const float* recv_scale,
                           const int32_t* expert_offset, const moe_weights* w, const void* x, void* ws,
                           size_t ws_bytes, void* stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (T < 0 || !rows_fit(cfg, T)) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if ((st = check_weights(cfg, w)) != MOE_OK) return st;
  if (!recv || !expert_offset || !ws) return MOE_ERR_INVALID_ARG;
  if (fp8(cfg) && !recv_scale) return MOE_ERR_INVALID_ARG;
  if (cfg->num_shared && !fp8(cfg) && !x) return MOE_ERR_INVALID_ARG;
  if (!all_aligned(recv, expert_offset, ws) || (recv_scale && !aligned16(recv_scale)) || (x && !aligned16(x)))
    return MOE_ERR_INVALID_ARG;
  if (ws_bytes < ffn_layout(cfg, T).total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  return gate_up_impl(cfg, T, recv, recv_scale, expert_offset, w, x, ws, (hipStream_t)stream);
}

moe_status moe_ffn_down(const moe_config* cfg, int32_t T, const int32_t* expert_offset, const moe_weights* w,
                        const void* ws, size_t ws_bytes, float* expert_out, float* shared_out, void* stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (T < 0 || !rows_fit(cfg, T)) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if ((st = check_weights(cfg, w)) != MOE_OK) return st;
  if (!expert_offset || !ws || !expert_out) return MOE_ERR_INVALID_ARG;
  if (cfg->num_shared && !shared_out) return MOE_ERR_INVALID_ARG;
  if (!all_aligned(expert_offset, ws, expert_out) || (shared_out && !aligned16(shared_out)))
    return MOE_ERR_INVALID_ARG;
  if (ws_bytes < ffn_layout(cfg, T).total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  return down_impl(cfg, T, expert_offset, w, ws, expert_out, shared_out, (hipStream_t)stream);
}

}  // extern "C"

namespace {

// The router GEMM above 16 tokens: a plain pass over one group that holds all
// T tokens (the slot the shared expert uses), with no routed groups and fp32
// output.
FfnParams router_params(const moe_config* c, int32_t T, const void* x, const void* w_router, float* logits) {
  const int E = c->num_experts, d = c->d_model;
  FfnParams r{};
  r.E = 0;       // no routed groups
  r.masked = 1;  // so no offsets array is read
  r.T = T;
  r.n_shared = 1;
  r.tiles_r = 0;
  r.tiles_s = E / 16;
  r.K_r = d; r.NW_r = E; r.Nout_r = E;
  r.s_act = static_cast<const uint8_t*>(x);
  r.s_w = static_cast<const uint8_t*>(w_router);
  r.K_s = d; r.NW_s = E; r.Nout_s = E;
  r.s_out = logits;
  return r;
}

// From 2048 bf16 tokens on (E a multiple of 128) the LDS-tiled kernel runs
// the router GEMM, reusing each weight tile across 128 tokens.
bool router_tiled(const moe_config* c, int64_t T) {
  return c->act_dtype == MOE_BF16 && T >= 2048 && c->num_experts % 128 == 0;
}

// With a workspace, bf16 router GEMMs of at least split_min_tokens tokens (E
// a multiple of 128) run on the LDS-tiled kernel with the reduction split.
// Measured against the unsplit path (DeepSeek-V3 shapes, d 7168: 256 tokens
// 27.6 against 30.1 us, 512 29.0 / 40.4, 1024 29.4 / 66.5, 4096 38.4 /
// 108.1; Qwen3 shapes, d 2048: 512 19.8 against 19.2 us, 1024 19.5 / 24.2,
// 4096 21.3 / 29.7).
int64_t split_min_tokens(const moe_config* c) { return c->d_model >= 4096 ? 256 : 1024; }

// Parts of the tiled router GEMM's reduction when a workspace is given: the
// pass has only ceil(T/128) x E/WR tiles (WR = 256 weight rows when E % 256
// == 0, else 128), so the K-steps are split until about 256 items run, into
// at most 16 parts of at least 8 steps each.  1: not split.
int router_split(const moe_config* c, int64_t T) {
  if (c->act_dtype != MOE_BF16 || T < split_min_tokens(c) || c->num_experts % 128) return 1;
  const int E = c->num_experts;
  const int64_t tiles = (T + 127) / 128 * (E / (E % 256 == 0 ? 256 : 128));
  int64_t P = 256 / tiles;
  if (P > 16) P = 16;
  if (P > c->d_model / 64 / 8) P = c->d_model / 64 / 8;
  return P < 2 ? 1 : (int)P;
}

moe_status router_check(const moe_config* cfg, int32_t T, const void* x, const void* w_router, const float* logits) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (T < 0) return MOE_ERR_INVALID_ARG;
  if (cfg->num_experts % 64) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !w_router || !logits || !all_aligned(x, w_router, logits)) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

}  // namespace

extern "C" {

// The router GEMM: dot products for up to 16 tokens (one workgroup per
// expert); above that the plain pass of router_params: the weight-streaming
// kernel up to 2047 tokens, the LDS-tiled kernel from 2048 bf16 tokens on.
// The tiled kernel has only T/128 x E/256 items here, so below that it
// leaves most CUs idle (512 tokens: 111 us tiled), and without a workspace it
// walks all of K in each item (moe_router_logits_ws splits it).
moe_status moe_router_logits(const moe_config* cfg, int32_t T, const void* x, const void* w_router,
                             float* logits, void* stream) {
  const moe_status st = router_check(cfg, T, x, w_router, logits);
  if (st != MOE_OK || T == 0) return st;
  if (router_gemv_fits(T, cfg->d_model, cfg->act_dtype))
    return hip_status(launch_router_gemv(x, w_router, logits, T, cfg->num_experts, cfg->d_model, cfg->act_dtype,
                                         (hipStream_t)stream));
  const FfnParams r = router_params(cfg, T, x, w_router, logits);
  if (router_tiled(cfg, T)) return hip_status(launch_gemm_tiled(r, false, 0, (hipStream_t)stream));
  return hip_status(launch_router_gemm(r, cfg->act_dtype, (hipStream_t)stream));
}

size_t moe_router_workspace_size(const moe_config* cfg, int32_t max_tokens) {
  if (check_config(cfg) != MOE_OK || max_tokens < 0) return 0;
  // P(T) T is largest at the last token count of some tile count
  size_t best = 0;
  for (int64_t tiles = 1; tiles * 128 - 127 <= max_tokens; ++tiles) {
    const int64_t T = tiles * 128 < max_tokens ? tiles * 128 : max_tokens;
    const int P = router_split(cfg, T);
    if (P < 2) {
      if (T >= split_min_tokens(cfg)) break;  // P does not grow with T
      continue;
    }
    const size_t b = (size_t)P * (size_t)T * cfg->num_experts * sizeof(float);
    best = b > best ? b : best;
  }
  return best;
}

moe_status moe_router_logits_ws(const moe_config* cfg, int32_t T, const void* x, const void* w_router,
                                float* logits, void* ws, size_t ws_bytes, void* stream) {
  const moe_status st = router_check(cfg, T, x, w_router, logits);
  if (st != MOE_OK || T == 0) return st;
  const int P = router_split(cfg, T);
  if (P < 2) return moe_router_logits(cfg, T, x, w_router, logits, stream);
  const size_t need = (size_t)P * (size_t)T * cfg->num_experts * sizeof(float);
  if (ws_bytes < need) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (!ws || !aligned16(ws)) return MOE_ERR_INVALID_ARG;
  FfnParams r = router_params(cfg, T, x, w_router, static_cast<float*>(ws));
  r.ksplit = P;
  const hipError_t e = launch_gemm_tiled(r, false, 0, (hipStream_t)stream);
  if (e != hipSuccess) return hip_status(e);
  return hip_status(launch_router_split_sum(static_cast<const float*>(ws), logits, (long long)T * cfg->num_experts, P,
                                            (hipStream_t)stream));
}

moe_status moe_combine(const moe_config* cfg, int32_t T, const float* expert_out, const int32_t* row_of,
                       const float* topk_w, const float* shared_out, void* y, int32_t* expert_count,
                       void* stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (T < 0 || !rows_fit(cfg, T)) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!expert_out || !row_of || !topk_w || !y || !expert_count) return MOE_ERR_INVALID_ARG;
  if (!all_aligned(expert_out, row_of, topk_w, y, expert_count) || (shared_out && !aligned16(shared_out)))
    return MOE_ERR_INVALID_ARG;
  return combine_impl(cfg, T, expert_out, row_of, topk_w, shared_out, y, expert_count, (hipStream_t)stream);
}

moe_status moe_layer(const moe_config* cfg, int32_t T, const void* x, const float* logits, const float* bias,
                     const moe_weights* w, void* y, void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (T < 0 || !rows_fit(cfg, T)) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if ((st = check_weights(cfg, w)) != MOE_OK) return st;
  if (!x || !logits || !y || !ws) return MOE_ERR_INVALID_ARG;
  if (!all_aligned(x, logits, y, ws) || (bias && !aligned16(bias))) return MOE_ERR_INVALID_ARG;
  const LayerLayout L = layer_layout(cfg, T);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t s = (hipStream_t)stream;
  uint8_t* b = static_cast<uint8_t*>(ws);
  int32_t* count = reinterpret_cast<int32_t*>(b + L.count);
  int32_t* idx = reinterpret_cast<int32_t*>(b + L.idx);
  float* tw = reinterpret_cast<float*>(b + L.w);
  int32_t* ticket = reinterpret_cast<int32_t*>(b + L.ticket);
  int32_t* row_of = reinterpret_cast<int32_t*>(b + L.row_of);
  int32_t* offset = reinterpret_cast<int32_t*>(b + L.offset);
  void* recv = b + L.recv;
  float* recv_scale = fp8(cfg) ? reinterpret_cast<float*>(b + L.recv_scale) : nullptr;
  float* eout = reinterpret_cast<float*>(b + L.eout);
  float* sout = cfg->num_shared ? reinterpret_cast<float*>(b + L.sout) : nullptr;
  void* ffn_ws = b + L.ffn;
  if (masked(cfg)) {
    // route and dispatch in one launch; the GEMMs read the counters in
    // place of offsets
    RouteParams rp = route_params(cfg, T, logits, bias, idx, tw, count, nullptr);
    fuse_dispatch(rp, cfg, x, recv, recv_scale, row_of);
    if (cfg->num_shared && !use_tiled(cfg, T)) {
      const FfnParams a = gate_up_params(cfg, T, recv, recv_scale, count, w, x, ffn_ws);
      if (route_shared_supported(a, cfg->weight_dtype)) {
        if ((st = hip_status(launch_route_shared(rp, a, cfg->weight_dtype, s))) != MOE_OK) return st;
        FfnParams routed = a;
        routed.n_shared = 0;
        if ((st = hip_status(launch_ffn(routed, cfg->weight_dtype, true, (long long)T * cfg->top_k,
                                        max_groups_of(cfg, T), s))) != MOE_OK)
          return st;
        if ((st = down_impl(cfg, T, count, w, ffn_ws, eout, sout, s)) != MOE_OK) return st;
        return combine_impl(cfg, T, eout, row_of, tw, sout, y, count, s);
      }
    }
    if ((st = hip_status(launch_route(rp, s))) != MOE_OK) return st;
    if ((st = ffn_impl(cfg, T, recv, recv_scale, count, w, x, eout, sout, ffn_ws, s)) != MOE_OK) return st;
    return combine_impl(cfg, T, eout, row_of, tw, sout, y, count, s);
  }
  if (cfg->num_shared && !use_tiled(cfg, T)) {
    // The shared expert needs no routing: its gate/up pass streams its
    // weights in the router's launch, and the routed pass follows dispatch.
    const FfnParams a = gate_up_params(cfg, T, recv, recv_scale, offset, w, x, ffn_ws);
    if (route_shared_supported(a, cfg->weight_dtype)) {
      const RouteParams rp = route_params(cfg, T, logits, bias, idx, tw, count, ticket);
      if ((st = hip_status(launch_route_shared(rp, a, cfg->weight_dtype, s))) != MOE_OK) return st;
      if ((st = dispatch_impl(cfg, T, x, idx, count, ticket, recv, recv_scale, offset, row_of, s)) != MOE_OK)
        return st;
      FfnParams routed = a;
      routed.n_shared = 0;
      if ((st = hip_status(launch_ffn(routed, cfg->weight_dtype, true, (long long)T * cfg->top_k,
                                      max_groups_of(cfg, T), s))) != MOE_OK)
        return st;
      if ((st = down_impl(cfg, T, offset, w, ffn_ws, eout, sout, s)) != MOE_OK) return st;
      return combine_impl(cfg, T, eout, row_of, tw, sout, y, count, s);
    }
  }
  if ((st = route_impl(cfg, T, logits, bias, idx, tw, count, ticket, s)) != MOE_OK) return st;
  if ((st = dispatch_impl(cfg, T, x, idx, count, ticket, recv, recv_scale, offset, row_of, s)) != MOE_OK) return st;
  if ((st = ffn_impl(cfg, T, recv, recv_scale, offset, w, x, eout, sout, ffn_ws, s)) != MOE_OK) return st;
  return combine_impl(cfg, T, eout, row_of, tw, sout, y, count, s);
}

size_t moe_fused_workspace_size(const moe_config* cfg, int32_t max_tokens) {
  if (check_config(cfg) != MOE_OK || max_tokens < 0) return 0;
  return fused_layout(cfg, max_tokens).total;
}

int32_t moe_fused_supported(const moe_config* cfg, int32_t T) {
  return check_config(cfg) == MOE_OK && fused_ok(cfg, T) ? 1 : 0;
}

moe_status moe_layer_fused(const moe_config* cfg, int32_t T, const void* x, const float* logits, const void* w_router,
                           const float* bias, const moe_weights* w, void* y, void* ws, size_t ws_bytes,
                           void* stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (T < 0) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if ((logits == nullptr) == (w_router == nullptr)) return MOE_ERR_INVALID_ARG;
  if ((st = check_weights(cfg, w)) != MOE_OK) return st;
  if (!x || !y || !ws) return MOE_ERR_INVALID_ARG;
  if (!all_aligned(x, y, ws) || (logits && !aligned16(logits)) || (w_router && !aligned16(w_router)) ||
      (bias && !aligned16(bias)))
    return MOE_ERR_INVALID_ARG;
  if (!fused_ok(cfg, T)) return MOE_ERR_UNSUPPORTED;
  if (w_router && !router_gemv_fits(T, cfg->d_model, MOE_BF16)) return MOE_ERR_UNSUPPORTED;
  const FusedLayout L = fused_layout(cfg, T);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  const moe_config cc = compact_of(cfg);
  uint8_t* b = static_cast<uint8_t*>(ws);
  FusedParams fp{};
  float* lws = reinterpret_cast<float*>(b + L.logits);
  fp.r = route_params(&cc, T, w_router ? lws : logits, bias, nullptr, nullptr, nullptr, nullptr);
  fp.d = cc.d_model;
  fp.F = cc.d_ff;
  fp.ns = cc.num_shared ? 1 : 0;
  fp.Fs = fp.ns ? cc.d_ff_shared : 0;
  fp.x = static_cast<const uint16_t*>(x);
  fp.w_router = static_cast<const uint16_t*>(w_router);
  fp.logits_ws = lws;
  fp.w13 = static_cast<const uint16_t*>(w->w13);
  fp.w2 = static_cast<const uint16_t*>(w->w2);
  fp.ws13 = fp.ns ? static_cast<const uint16_t*>(w->ws13) : nullptr;
  fp.ws2 = fp.ns ? static_cast<const uint16_t*>(w->ws2) : nullptr;
  fp.h = reinterpret_cast<uint16_t*>(b + L.h);
  fp.y = static_cast<uint16_t*>(y);
  fp.sync = reinterpret_cast<int*>(b + L.sync);
  fp.bar0 = fp.sync + kFusedBarWords;
  fp.bar1 = fp.sync + 2 * kFusedBarWords;
  fp.err = fp.sync + 4;
  fp.spin_limit = kFusedSpinLimit;
  return hip_status(launch_fused(fp, (hipStream_t)stream));
}

const char* moe_status_string(moe_status status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: invalid argument";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: configuration not supported by the kernels";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL: workspace below the required size";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: a HIP launch failed";
    case MOE_ERR_SCRATCH_LIMIT: return "MOE_ERR_SCRATCH_LIMIT: the call needs more than the library's static scratch";
  }
  return "unknown moe_status";
}

}  // extern "C"
