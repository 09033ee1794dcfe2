// Kernel parameter blocks and launchers (internal to the library).
#pragma once

#include "moe_device.h"

namespace moe {

struct RouteParams {
  int T, E, k, n_group, topk_group, score_fn, weight_fn;
  float routed_scale;
  const float* logits;
  const float* bias;
  int* topk_idx;
  float* topk_w;
  int* expert_count;
  int* ticket;  // may be NULL when fuse is set
  // fuse: also write the token into its masked-layout rows (row e*T +
  // ticket; E4M3 codes and scales when quant, plus row E*T + t for the
  // shared expert when shared_rows) and row_of
  int fuse, d, act_dtype, quant, shared_rows;
  const void* x;
  void* recv;
  float* recv_scale;
  int* row_of;
};

struct DispatchParams {
  int T, E, k, d, act_dtype;
  int quant;        // write E4M3 codes + per-128 scales
  int shared_rows;  // also write rows routed_rows + t for the shared expert (quant only)
  int masked;       // masked layout: row e*T + ticket, no offsets
  int routed_rows;  // T*k (compact) or E*T (masked)
  const void* x;
  const int* topk_idx;
  const int* expert_count;
  const int* ticket;
  void* recv;
  float* recv_scale;
  int* expert_offset;
  int* row_of;
};

// One grouped GEMM pass over the dispatch layout.  Work item = (group, tile):
// groups are the experts with rows (ranked by index) and then the shared
// expert; a tile is 16*FW consecutive output columns.  GATED passes multiply
// the gate rows [c, c+16FW) and the up rows [Nout + c, ...) of the same
// weight matrix and write silu(gate) * up; plain passes write the product.
struct FfnParams {
  int E, T;
  // compact layout: [E+1] offsets, expert e's rows are [off[e], off[e+1]);
  // masked layout: [E] counts, expert e's rows are [e*T, e*T + cnt[e])
  const int* expert_offset;
  int masked;
  int n_shared;
  int tiles_r, tiles_s;
  // routed experts: activation rows [expert_offset[e], expert_offset[e+1])
  const uint8_t* act;
  const float* act_scale;  // E4M3 only: [rows][K_r/128]
  const uint8_t* w;        // [E][NW_r][K_r]
  const float* w_scale;    // E4M3 only: [E][NW_r/128][K_r/128]
  int K_r, NW_r, Nout_r;
  void* out;               // [rows][Nout_r]
  float* out_scale;        // E4M3 output only: [rows][Nout_r/128]
  // shared expert: activation rows [0, T)
  const uint8_t* s_act;
  const float* s_act_scale;
  const uint8_t* s_w;
  const float* s_w_scale;
  int K_s, NW_s, Nout_s;
  void* s_out;
  float* s_out_scale;
  // LDS-tiled plain pass with no routed groups only (the router GEMM): the
  // reduction is split into ksplit parts (<= 1: not split); part q writes its
  // fp32 partial sums to s_out + q * T * Nout_s
  int ksplit;
};

struct CombineParams {
  int T, E, k, d, act_dtype;
  int routed_rows;  // rows of expert_out: slots whose row_of lies outside contribute nothing
  const float* expert_out;
  const int* row_of;
  const float* topk_w;
  const float* shared_out;
  void* y;
  int* expert_count;
};

// The whole layer for a handful of tokens (bf16) in one persistent launch.
// r: the routing rule (r.logits: the layer's logits, or logits_ws when the
// launch computes them from x and w_router).  Weights as in moe_weights.  h:
// the SwiGLU activations handed from the gate/up pass to the down pass, row
// t*k + j for slot j of token t ([T*k][F]), then the shared expert's row t
// ([T][Fs]).  Words that are zero between calls (the last workgroup to count
// out zeroes them): sync[3], the exit count; bar0, bar1: the blocks
// (kFusedBarWords ints: counters and a release flag) of the barriers after
// the router GEMM and after the gate/up pass.  err: set to 1 when a bounded wait
// gives up (the results are then invalid).
struct FusedParams {
  RouteParams r;
  int d, F, Fs, ns;
  const uint16_t* x;
  const uint16_t* w_router;  // nullptr: r.logits is an input
  float* logits_ws;
  const uint16_t* w13;  // [E][2F][d]
  const uint16_t* w2;   // [E][d][F]
  const uint16_t* ws13; // [2Fs][d]
  const uint16_t* ws2;  // [d][Fs]
  uint16_t* h;
  uint16_t* y;
  int* sync;
  int* bar0;
  int* bar1;
  int* err;
  int spin_limit;
};

constexpr int kFusedBarWords = 1024;  // ints per barrier block (4 KB)

// Whether the fused launch covers a shape (T tokens, k slots each, E experts,
// model width d, expert widths F and Fs; Fs = 0 without a shared expert).
bool fused_shape_ok(int T, int k, int E, int d, int F, int Fs);
// Workgroups of the fused launch on the current device (one per CU), or 0.
int fused_grid();

hipError_t launch_route(const RouteParams& p, hipStream_t stream);
hipError_t launch_fused(const FusedParams& p, hipStream_t stream);
hipError_t launch_dispatch(const DispatchParams& p, hipStream_t stream);
// gated: gate/up + SwiGLU pass (output dtype: bf16, or E4M3 with scales for
// E4M3 weights, or f32); otherwise the down pass (f32 output).  routed_rows
// is T*k and max_groups bounds the experts with rows (both size the grid).
hipError_t launch_ffn(const FfnParams& p, int wdtype, bool gated, long long routed_rows, int max_groups,
                      hipStream_t stream);
hipError_t launch_combine(const CombineParams& p, hipStream_t stream);
// Router and the shared expert's gate/up pass in one launch (sp: the full
// gate/up pass parameters; only its shared expert is run).  Supported for
// bf16 weights whose gate/up launch shape has four waves per workgroup.
bool route_shared_supported(const FfnParams& sp, int wdtype);
hipError_t launch_route_shared(const RouteParams& rp, const FfnParams& sp, int wdtype, hipStream_t stream);
// LDS-tiled bf16 grouped GEMM for groups with many rows (prefill);
// max_token_tiles bounds the 128-row token tiles over the routed groups
// (sizes the persistent grid).  Needs K % 64 == 0 and Nout % 128 == 0.
// Resident workgroups of one kernel: per CU, CU count, and the dynamic LDS
// reserved to cap residency.  Launchers compute it once per kernel, on first
// use, into a const local static.
struct Residency {
  int per_cu = 1, cus = 0;
  size_t reserve = 0;
  bool ok = false;
};

hipError_t launch_gemm_tiled(const FfnParams& p, bool gated, long long max_token_tiles, hipStream_t stream);
// Router GEMM over one group holding all T tokens (the shared-expert slot),
// plain pass, fp32 out: one 16-column tile per item, K split KS ways inside
// the workgroup, so a small router weight still spreads over E/16 workgroups.
hipError_t launch_router_gemm(const FfnParams& p, int dtype, hipStream_t stream);
// Router GEMM for 1-16 tokens as dot products: one workgroup per expert, the
// reduction split over its four waves.  router_gemv_fits says whether the
// shape is covered (d up to 16384 bf16 / 8192 fp32).
bool router_gemv_fits(int T, int d, int dtype);
hipError_t launch_router_gemv(const void* x, const void* w, float* logits, int T, int E, int d, int dtype,
                              hipStream_t stream);
// logits[i] = sum of part[q][i] over q = 0 .. P-1 in that order (n values, n % 4 == 0)
hipError_t launch_router_split_sum(const float* part, float* logits, long long n, int P, hipStream_t stream);

// FfnParams::tiles_r / tiles_s count 16-column tiles; launch_ffn groups them
// into the work items of the launch shape it picks (a gated E4M3 pass always
// covers 128 columns per item, so each 1x128 block of h is quantised inside one
// workgroup).

}  // namespace moe
