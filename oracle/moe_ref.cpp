// Plain C++ CPU oracle of the MoE layer (test infrastructure only; see
// moe_ref.h for the sources and conventions).  Written to be checked by eye
// against the pages: every step is a loop over the definition, every dot
// product and reduction is accumulated in double in index order, and nothing
// is blocked, fused or reordered.  Threads only split independent output
// elements (a feature of one expert), so the thread count never changes a
// result.  Built with -ffp-contract=off: no multiply-add is fused.
#include "moe_ref.h"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <limits>
#include <thread>
#include <vector>

namespace {

const double kInf = std::numeric_limits<double>::infinity();
const float kInfF = std::numeric_limits<float>::infinity();

bool config_ok(const moe_ref_config* c) {
  if (!c) return false;
  const int E = c->num_experts, k = c->top_k, G = c->n_group, kg = c->topk_group;
  if (E < 1 || k < 1 || k > E || G < 1 || E % G || kg < 1 || kg > G || k > kg * (E / G)) return false;
  if (c->d_model < 1 || c->d_ff < 1) return false;
  if (c->num_shared && c->d_ff_shared < 1) return false;
  if (c->weight_dtype == MOE_REF_E4M3 && (c->d_model % 128 || c->d_ff % 128 ||
                                          (c->num_shared && c->d_ff_shared % 128)))
    return false;
  if (c->act_quant && (c->d_model % 128 || c->d_ff % 128 || (c->num_shared && c->d_ff_shared % 128)))
    return false;
  return true;
}

// Run fn(lo, hi) over [0, n) split into contiguous ranges, one per thread.
template <class Fn>
void parallel_for(int64_t n, int nthreads, Fn fn) {
  if (nthreads <= 0) nthreads = (int)std::thread::hardware_concurrency();
  if (nthreads < 1) nthreads = 1;
  if (nthreads > n) nthreads = (int)std::max<int64_t>(n, 1);
  if (nthreads == 1) {
    fn((int64_t)0, n);
    return;
  }
  std::vector<std::thread> pool;
  const int64_t chunk = (n + nthreads - 1) / nthreads;
  for (int i = 0; i < nthreads; ++i) {
    const int64_t lo = i * chunk, hi = std::min(n, lo + chunk);
    if (lo < hi) pool.emplace_back(fn, lo, hi);
  }
  for (auto& t : pool) t.join();
}

// ---------------------------------------------------------------------------
// Storage decoding
// ---------------------------------------------------------------------------

double bf16_value(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

double elem(const void* base, int dtype, int64_t i) {
  switch (dtype) {
    case MOE_REF_F32: return static_cast<const float*>(base)[i];
    case MOE_REF_BF16: return bf16_value(static_cast<const uint16_t*>(base)[i]);
    case MOE_REF_F64: return static_cast<const double*>(base)[i];
    default: return std::nan("");
  }
}

// One weight matrix [rows][cols]; E4M3 codes carry one fp32 scale per
// 128 x 128 block.
struct Mat {
  const void* p;
  const float* s;
  int dtype;
  int64_t rows, cols;

  void row(int64_t r, double* out) const {
    for (int64_t c = 0; c < cols; ++c) {
      if (dtype == MOE_REF_E4M3) {
        const uint8_t code = static_cast<const uint8_t*>(p)[r * cols + c];
        out[c] = moe_ref_e4m3_decode(code) * (double)s[(r / 128) * (cols / 128) + c / 128];
      } else {
        out[c] = elem(p, dtype, r * cols + c);
      }
    }
  }
};

int64_t elem_bytes(int dtype) {
  return dtype == MOE_REF_F32 ? 4 : dtype == MOE_REF_BF16 ? 2 : dtype == MOE_REF_E4M3 ? 1 : 8;
}

Mat expert_mat(const moe_ref_config* c, const moe_ref_weights* w, int e, bool up) {
  const int64_t d = c->d_model, F = c->d_ff;
  const int64_t rows = up ? 2 * F : d, cols = up ? d : F;
  const uint8_t* base = static_cast<const uint8_t*>(up ? w->w13 : w->w2);
  const float* sc = up ? w->w13_scale : w->w2_scale;
  Mat m{base + (size_t)e * rows * cols * elem_bytes(c->weight_dtype), nullptr, c->weight_dtype, rows, cols};
  if (c->weight_dtype == MOE_REF_E4M3) m.s = sc + (size_t)e * (rows / 128) * (cols / 128);
  return m;
}

Mat shared_mat(const moe_ref_config* c, const moe_ref_weights* w, bool up) {
  const int64_t d = c->d_model, Fs = c->d_ff_shared;
  Mat m{up ? w->ws13 : w->ws2, nullptr, c->weight_dtype, up ? 2 * Fs : d, up ? d : Fs};
  if (c->weight_dtype == MOE_REF_E4M3) m.s = up ? w->ws13_scale : w->ws2_scale;
  return m;
}

double dot(const double* a, const double* b, int64_t n) {
  double s = 0.0;
  for (int64_t i = 0; i < n; ++i) s += a[i] * b[i];
  return s;
}

// Values code * scale of fp32 rows quantised per 1x128 block.
void quant_dequant_rows(int64_t n, int64_t d, double* rows) {
  std::vector<float> f(d);
  std::vector<uint8_t> codes(d);
  std::vector<float> scales(d / 128);
  for (int64_t r = 0; r < n; ++r) {
    for (int64_t i = 0; i < d; ++i) f[i] = (float)rows[r * d + i];
    moe_ref_quantize_rows(1, d, f.data(), codes.data(), scales.data());
    for (int64_t i = 0; i < d; ++i) rows[r * d + i] = moe_ref_e4m3_decode(codes[i]) * (double)scales[i / 128];
  }
}

// One SwiGLU expert on n rows a [n][d]: out[r] = W2 (silu(Wg a_r) * (Wu a_r)).
void swiglu(const moe_ref_config* c, const Mat& w13, const Mat& w2, const double* a_in, int64_t n,
            double* out, int nthreads) {
  const int64_t d = w13.cols, F = w13.rows / 2;
  std::vector<double> a(a_in, a_in + n * d);
  if (c->act_quant) quant_dequant_rows(n, d, a.data());
  std::vector<double> h((size_t)n * F);
  parallel_for(F, nthreads, [&](int64_t lo, int64_t hi) {
    std::vector<double> g(d), u(d);
    for (int64_t i = lo; i < hi; ++i) {
      w13.row(i, g.data());
      w13.row(F + i, u.data());
      for (int64_t r = 0; r < n; ++r) {
        const double gate = dot(g.data(), &a[r * d], d);
        const double up = dot(u.data(), &a[r * d], d);
        h[r * F + i] = gate * (1.0 / (1.0 + std::exp(-gate))) * up;
      }
    }
  });
  if (c->act_quant) {
    // h is rounded to fp32 before its 1x128 quantisation
    quant_dequant_rows(n, F, h.data());
  }
  parallel_for(d, nthreads, [&](int64_t lo, int64_t hi) {
    std::vector<double> wd(F);
    for (int64_t o = lo; o < hi; ++o) {
      w2.row(o, wd.data());
      for (int64_t r = 0; r < n; ++r) out[r * d + o] = dot(wd.data(), &h[r * F], F);
    }
  });
}

float key_of(const moe_ref_config* c, float logit, const float* bias, int e) {
  float k;
  if (c->score_fn == 1) {
    const float s = (float)(1.0 / (1.0 + std::exp(-(double)logit)));
    k = bias ? s + bias[e] : s;
  } else {
    k = logit;
  }
  return std::isnan(k) ? -kInfF : k;
}

// Candidate a ranks before b: larger value, then lower index.
bool better(double va, int ia, double vb, int ib) { return va > vb || (va == vb && ia < ib); }

// Group scores and eligibility of one token's keys.
void groups_of(const moe_ref_config* c, const float* keys, std::vector<float>& gs, std::vector<char>& elig) {
  const int E = c->num_experts, G = c->n_group, gsize = E / G;
  elig.assign(E, 1);
  gs.clear();
  if (G == 1) return;
  gs.resize(G);
  for (int q = 0; q < G; ++q) {
    // the two largest keys of the group (by value; NaN keys are already -inf)
    float b1 = -kInfF, b2 = -kInfF;
    int i1 = -1;
    for (int j = 0; j < gsize; ++j) {
      const float v = keys[q * gsize + j];
      if (i1 < 0 || v > b1) { b1 = v; i1 = j; }
    }
    for (int j = 0; j < gsize; ++j) {
      if (j == i1) continue;
      const float v = keys[q * gsize + j];
      if (v > b2) b2 = v;
    }
    float s = gsize == 1 ? b1 : b1 + b2;
    gs[q] = std::isnan(s) ? -kInfF : s;
  }
  // the topk_group best groups, by repeated selection of the best remaining
  std::vector<char> chosen(G, 0);
  for (int n = 0; n < c->topk_group; ++n) {
    int best = -1;
    for (int q = 0; q < G; ++q)
      if (!chosen[q] && (best < 0 || better(gs[q], q, gs[best], best))) best = q;
    chosen[best] = 1;
  }
  for (int e = 0; e < E; ++e) elig[e] = chosen[e / gsize];
}

}  // namespace

extern "C" {

double moe_ref_e4m3_decode(uint8_t code) {
  const int sign = code >> 7, ex = (code >> 3) & 15, m = code & 7;
  if (ex == 15 && m == 7) return std::nan("");
  const double mag = ex == 0 ? m * std::ldexp(1.0, -9) : (1.0 + m / 8.0) * std::ldexp(1.0, ex - 7);
  return sign ? -mag : mag;
}

uint8_t moe_ref_e4m3_encode(float v) {
  if (std::isnan(v)) return 0x7F;
  const double a = std::fabs((double)v);
  int code;
  if (a >= 448.0) {
    code = 126;
  } else {
    // the nearest of the 127 non-negative finite values; ties to the even code
    code = 0;
    double best = kInf;
    for (int cc = 0; cc <= 126; ++cc) {
      const double dist = std::fabs(a - moe_ref_e4m3_decode((uint8_t)cc));
      if (dist < best || (dist == best && (cc & 1) == 0)) {
        best = dist;
        code = cc;
      }
    }
  }
  if (v < 0 && code != 0) code |= 0x80;
  return (uint8_t)code;
}

int moe_ref_quantize_rows(int64_t n, int64_t d, const float* x, uint8_t* codes, float* scales) {
  if (n < 0 || d % 128) return -1;
  for (int64_t r = 0; r < n; ++r)
    for (int64_t b = 0; b < d / 128; ++b) {
      const float* blk = x + r * d + b * 128;
      float amax = 0.f;
      for (int i = 0; i < 128; ++i) amax = std::max(amax, std::fabs(blk[i]));
      const float scale = amax > 0.f ? amax / 448.0f : 1.0f;
      scales[r * (d / 128) + b] = scale;
      for (int i = 0; i < 128; ++i) codes[r * d + b * 128 + i] = moe_ref_e4m3_encode(blk[i] / scale);
    }
  return 0;
}

int moe_ref_keys(const moe_ref_config* c, int32_t T, const float* logits, const float* bias, float* keys) {
  if (!config_ok(c) || T < 0) return -1;
  const int E = c->num_experts;
  for (int64_t t = 0; t < T; ++t)
    for (int e = 0; e < E; ++e) keys[t * E + e] = key_of(c, logits[t * E + e], c->score_fn == 1 ? bias : nullptr, e);
  return 0;
}

int moe_ref_gate_weights(const moe_ref_config* c, int32_t T, const float* logits, const int32_t* topk_idx,
                         double* topk_w) {
  if (!config_ok(c) || T < 0) return -1;
  const int E = c->num_experts, k = c->top_k;
  std::vector<double> sel(k);
  for (int64_t t = 0; t < T; ++t) {
    const float* l = logits + t * E;
    if (c->score_fn == 0) {
      // softmax over every expert (max subtracted; NaN propagates)
      double m = -kInf;
      bool nan = false;
      for (int e = 0; e < E; ++e) {
        if (std::isnan(l[e])) nan = true;
        else m = std::max(m, (double)l[e]);
      }
      if (nan) m = std::nan("");
      double z = 0.0;
      for (int e = 0; e < E; ++e) z += std::exp((double)l[e] - m);
      for (int j = 0; j < k; ++j) sel[j] = std::exp((double)l[topk_idx[t * k + j]] - m) / z;
    } else {
      for (int j = 0; j < k; ++j) sel[j] = 1.0 / (1.0 + std::exp(-(double)l[topk_idx[t * k + j]]));
    }
    if (c->weight_fn == 0) {
      double s = 0.0;
      for (int j = 0; j < k; ++j) s += sel[j];
      for (int j = 0; j < k; ++j) topk_w[t * k + j] = sel[j] / s * c->routed_scale;
    } else {
      double m = -kInf;
      bool nan = false;
      for (int j = 0; j < k; ++j) {
        if (std::isnan(sel[j])) nan = true;
        else m = std::max(m, sel[j]);
      }
      if (nan) m = std::nan("");
      double z = 0.0;
      for (int j = 0; j < k; ++j) z += std::exp(sel[j] - m);
      for (int j = 0; j < k; ++j) topk_w[t * k + j] = std::exp(sel[j] - m) / z * c->routed_scale;
    }
  }
  return 0;
}

int moe_ref_route(const moe_ref_config* c, int32_t T, const float* logits, const float* bias, int32_t* topk_idx,
                  double* topk_w) {
  if (!config_ok(c) || T < 0) return -1;
  const int E = c->num_experts, k = c->top_k;
  std::vector<float> keys((size_t)E);
  std::vector<float> gs;
  std::vector<char> elig, taken;
  for (int64_t t = 0; t < T; ++t) {
    moe_ref_keys(c, 1, logits + t * E, bias, keys.data());
    groups_of(c, keys.data(), gs, elig);
    // top-k among the eligible experts, by repeated selection of the best
    taken.assign(E, 0);
    for (int j = 0; j < k; ++j) {
      int best = -1;
      for (int e = 0; e < E; ++e)
        if (elig[e] && !taken[e] && (best < 0 || better(keys[e], e, keys[best], best))) best = e;
      taken[best] = 1;
      topk_idx[t * k + j] = best;
    }
  }
  return moe_ref_gate_weights(c, T, logits, topk_idx, topk_w);
}

int moe_ref_margins(const moe_ref_config* c, int32_t T, const float* logits, const float* bias, double* gap) {
  if (!config_ok(c) || T < 0) return -1;
  const int E = c->num_experts, k = c->top_k, G = c->n_group, kg = c->topk_group;
  std::vector<float> keys((size_t)E);
  std::vector<float> gs;
  std::vector<char> elig;
  for (int64_t t = 0; t < T; ++t) {
    moe_ref_keys(c, 1, logits + t * E, bias, keys.data());
    groups_of(c, keys.data(), gs, elig);
    // eligible keys in rank order
    std::vector<int> order;
    for (int e = 0; e < E; ++e)
      if (elig[e]) order.push_back(e);
    std::stable_sort(order.begin(), order.end(),
                     [&](int a, int b) { return better(keys[a], a, keys[b], b); });
    double g = kInf;
    if ((int)order.size() > k) g = (double)keys[order[k - 1]] - (double)keys[order[k]];
    if (G > 1 && kg < G) {
      std::vector<int> go(G);
      for (int q = 0; q < G; ++q) go[q] = q;
      std::stable_sort(go.begin(), go.end(), [&](int a, int b) { return better(gs[a], a, gs[b], b); });
      const double gg = (double)gs[go[kg - 1]] - (double)gs[go[kg]];
      if (std::isnan(gg) || gg < g) g = gg;  // a NaN gap (infinite scores on both sides) is a tie
    }
    gap[t] = std::isnan(g) ? 0.0 : g;
  }
  return 0;
}

int moe_ref_dispatch(const moe_ref_config* c, int32_t T, const int32_t* topk_idx, int32_t* counts,
                     int32_t* offsets, int32_t* row_of, int32_t* token_of_row) {
  if (!config_ok(c) || T < 0) return -1;
  const int E = c->num_experts, k = c->top_k;
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t i = 0; i < (int64_t)T * k; ++i) {
    const int e = topk_idx[i];
    if (e < 0 || e >= E) return -1;
    ++counts[e];
  }
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  std::vector<int32_t> fill(offsets, offsets + E);
  for (int64_t t = 0; t < T; ++t)
    for (int j = 0; j < k; ++j) {
      const int r = fill[topk_idx[t * k + j]]++;
      row_of[t * k + j] = r;
      token_of_row[r] = (int32_t)t;
    }
  return 0;
}

int moe_ref_gather(const moe_ref_config* c, int32_t T, const void* x, const int32_t* token_of_row, double* recv) {
  if (!config_ok(c) || T < 0) return -1;
  const int64_t d = c->d_model;
  for (int64_t r = 0; r < (int64_t)T * c->top_k; ++r)
    for (int64_t i = 0; i < d; ++i) recv[r * d + i] = elem(x, c->act_dtype, token_of_row[r] * d + i);
  return 0;
}

int moe_ref_expert_ffn(const moe_ref_config* c, int32_t T, const double* recv, const int32_t* offsets,
                       const moe_ref_weights* w, const void* x, double* expert_out, double* shared_out,
                       int32_t nthreads) {
  if (!config_ok(c) || T < 0 || !w) return -1;
  const int64_t d = c->d_model;
  for (int e = 0; e < c->num_experts; ++e) {
    const int64_t lo = offsets[e], hi = offsets[e + 1];
    if (hi == lo) continue;  // an expert with no rows reads none of its weights
    swiglu(c, expert_mat(c, w, e, true), expert_mat(c, w, e, false), recv + lo * d, hi - lo, expert_out + lo * d,
           nthreads);
  }
  if (c->num_shared && shared_out) {
    std::vector<double> xs((size_t)T * d);
    for (int64_t i = 0; i < (int64_t)T * d; ++i) xs[i] = elem(x, c->act_dtype, i);
    swiglu(c, shared_mat(c, w, true), shared_mat(c, w, false), xs.data(), T, shared_out, nthreads);
  }
  return 0;
}

int moe_ref_combine(const moe_ref_config* c, int32_t T, const double* expert_out, const int32_t* row_of,
                    const double* topk_w, const double* shared_out, double* y) {
  if (!config_ok(c) || T < 0) return -1;
  const int64_t d = c->d_model;
  const int k = c->top_k;
  for (int64_t t = 0; t < T; ++t)
    for (int64_t o = 0; o < d; ++o) {
      double acc = 0.0;
      for (int j = 0; j < k; ++j) acc += topk_w[t * k + j] * expert_out[(int64_t)row_of[t * k + j] * d + o];
      if (shared_out) acc += shared_out[t * d + o];
      y[t * d + o] = acc;
    }
  return 0;
}

int moe_ref_layer(const moe_ref_config* c, int32_t T, const void* x, const float* logits, const float* bias,
                  const moe_ref_weights* w, const int32_t* topk_idx, const double* topk_w, double* y,
                  int32_t nthreads) {
  if (!config_ok(c) || T < 0 || !w || (!logits && !topk_idx)) return -1;
  const int E = c->num_experts, k = c->top_k;
  const int64_t d = c->d_model, tk = (int64_t)T * k;
  std::vector<int32_t> idx((size_t)tk);
  std::vector<double> wt((size_t)tk);
  if (topk_idx) {
    std::copy(topk_idx, topk_idx + tk, idx.begin());
    std::copy(topk_w, topk_w + tk, wt.begin());
  } else if (moe_ref_route(c, T, logits, bias, idx.data(), wt.data())) {
    return -1;
  }
  std::vector<int32_t> counts(E), offsets(E + 1), row_of((size_t)tk), tok((size_t)tk);
  if (moe_ref_dispatch(c, T, idx.data(), counts.data(), offsets.data(), row_of.data(), tok.data())) return -1;
  std::vector<double> recv((size_t)tk * d), eout((size_t)tk * d);
  moe_ref_gather(c, T, x, tok.data(), recv.data());
  std::vector<double> sout(c->num_shared ? (size_t)T * d : 0);
  moe_ref_expert_ffn(c, T, recv.data(), offsets.data(), w, x, eout.data(), c->num_shared ? sout.data() : nullptr,
                     nthreads);
  return moe_ref_combine(c, T, eout.data(), row_of.data(), wt.data(), c->num_shared ? sout.data() : nullptr, y);
}

int moe_ref_dense_token(const moe_ref_config* c, const void* x_row, const int32_t* idx_row, const double* w_row,
                        const moe_ref_weights* w, double* y_row) {
  if (!config_ok(c) || !w) return -1;
  const int64_t d = c->d_model;
  std::vector<double> xt(d), out(d);
  for (int64_t i = 0; i < d; ++i) xt[i] = elem(x_row, c->act_dtype, i);
  for (int64_t o = 0; o < d; ++o) y_row[o] = 0.0;
  for (int j = 0; j < c->top_k; ++j) {
    const int e = idx_row[j];
    if (e < 0 || e >= c->num_experts) return -1;
    swiglu(c, expert_mat(c, w, e, true), expert_mat(c, w, e, false), xt.data(), 1, out.data(), 1);
    for (int64_t o = 0; o < d; ++o) y_row[o] += w_row[j] * out[o];
  }
  if (c->num_shared) {
    swiglu(c, shared_mat(c, w, true), shared_mat(c, w, false), xt.data(), 1, out.data(), 1);
    for (int64_t o = 0; o < d; ++o) y_row[o] += out[o];
  }
  return 0;
}

int moe_ref_router_logits(const moe_ref_config* c, int32_t T, const void* x, const void* w_router,
                          double* logits) {
  if (!config_ok(c) || T < 0) return -1;
  const int E = c->num_experts;
  const int64_t d = c->d_model;
  for (int64_t t = 0; t < T; ++t)
    for (int e = 0; e < E; ++e) {
      double s = 0.0;
      for (int64_t i = 0; i < d; ++i) s += elem(x, c->act_dtype, t * d + i) * elem(w_router, c->act_dtype, e * d + i);
      logits[t * E + e] = s;
    }
  return 0;
}

}  // extern "C"
