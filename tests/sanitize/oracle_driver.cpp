// Drives the C++ oracle (oracle/moe_ref.cpp) through every entry point on
// tiny layers, for a build with AddressSanitizer and UndefinedBehavior-
// Sanitizer: any out-of-bounds access, use of uninitialised heap memory
// through a bad index, signed overflow or misaligned access aborts the run.
// Inputs are fixed pseudo-random test data (a 64-bit LCG); the values do not
// matter, only that every code path runs.  Exit status 0 = clean.
#include <cmath>
#include <cstdio>
#include <cstring>
#include <vector>

#include "moe_ref.h"

namespace {

uint64_t g_state = 0x2545F4914F6CDD1DULL;
float uniform() {  // in [-1, 1)
  g_state = g_state * 6364136223846793005ULL + 1442695040888963407ULL;
  return (float)((g_state >> 40) & 0xFFFFFF) / (float)(1 << 23) - 1.0f;
}
uint16_t to_bf16(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

int fails = 0;
void check(int rc, int want, const char* what) {
  if (rc != want) {
    std::printf("FAIL %s: returned %d, expected %d\n", what, rc, want);
    ++fails;
  }
}

// One layer configuration through route, dispatch, gather, expert FFN,
// combine, the whole layer, the dense per-token path and the margins.
void run_case(const moe_ref_config& c, int T) {
  const int E = c.num_experts, k = c.top_k, d = c.d_model, F = c.d_ff, Fs = c.d_ff_shared;
  const bool e4m3 = c.weight_dtype == MOE_REF_E4M3;
  std::vector<float> logits((size_t)T * E), bias(E), xf((size_t)T * d);
  for (auto& v : logits) v = uniform();
  for (auto& v : bias) v = 0.1f * uniform();
  for (auto& v : xf) v = uniform();
  std::vector<uint16_t> xb(xf.size());
  for (size_t i = 0; i < xf.size(); ++i) xb[i] = to_bf16(xf[i]);
  const void* x = c.act_dtype == MOE_REF_BF16 ? (const void*)xb.data() : (const void*)xf.data();

  const size_t n13 = (size_t)E * 2 * F * d, n2 = (size_t)E * d * F, ns13 = (size_t)2 * Fs * d, ns2 = (size_t)d * Fs;
  std::vector<float> f13(n13), f2(n2), fs13(ns13), fs2(ns2);
  for (auto* v : {&f13, &f2, &fs13, &fs2})
    for (auto& e : *v) e = 0.05f * uniform();
  std::vector<uint16_t> b13(n13), b2(n2), bs13(ns13), bs2(ns2);
  std::vector<uint8_t> q13(n13), q2(n2), qs13(ns13), qs2(ns2);
  for (size_t i = 0; i < n13; ++i) { b13[i] = to_bf16(f13[i]); q13[i] = moe_ref_e4m3_encode(f13[i] * 64.f); }
  for (size_t i = 0; i < n2; ++i) { b2[i] = to_bf16(f2[i]); q2[i] = moe_ref_e4m3_encode(f2[i] * 64.f); }
  for (size_t i = 0; i < ns13; ++i) { bs13[i] = to_bf16(fs13[i]); qs13[i] = moe_ref_e4m3_encode(fs13[i] * 64.f); }
  for (size_t i = 0; i < ns2; ++i) { bs2[i] = to_bf16(fs2[i]); qs2[i] = moe_ref_e4m3_encode(fs2[i] * 64.f); }
  std::vector<float> sc13((size_t)E * (2 * F / 128) * (d / 128), 1.f / 64), sc2((size_t)E * (d / 128) * (F / 128), 1.f / 64);
  std::vector<float> scs13((size_t)(2 * Fs / 128) * (d / 128) + 1, 1.f / 64), scs2((size_t)(d / 128) * (Fs / 128) + 1, 1.f / 64);
  moe_ref_weights w{};
  if (e4m3) {
    w = {q13.data(), q2.data(), c.num_shared ? qs13.data() : nullptr, c.num_shared ? qs2.data() : nullptr,
         sc13.data(), sc2.data(), c.num_shared ? scs13.data() : nullptr, c.num_shared ? scs2.data() : nullptr};
  } else if (c.weight_dtype == MOE_REF_BF16) {
    w = {b13.data(), b2.data(), c.num_shared ? bs13.data() : nullptr, c.num_shared ? bs2.data() : nullptr,
         nullptr, nullptr, nullptr, nullptr};
  } else {
    w = {f13.data(), f2.data(), c.num_shared ? fs13.data() : nullptr, c.num_shared ? fs2.data() : nullptr,
         nullptr, nullptr, nullptr, nullptr};
  }

  std::vector<float> keys((size_t)T * E);
  check(moe_ref_keys(&c, T, logits.data(), bias.data(), keys.data()), 0, "keys");
  std::vector<int32_t> idx((size_t)T * k + 1);
  std::vector<double> tw((size_t)T * k + 1), tw2((size_t)T * k + 1), gap((size_t)T + 1);
  check(moe_ref_route(&c, T, logits.data(), bias.data(), idx.data(), tw.data()), 0, "route");
  check(moe_ref_gate_weights(&c, T, logits.data(), idx.data(), tw2.data()), 0, "gate_weights");
  check(moe_ref_margins(&c, T, logits.data(), bias.data(), gap.data()), 0, "margins");
  std::vector<int32_t> counts(E), offsets(E + 1), row_of((size_t)T * k + 1), tok((size_t)T * k + 1);
  check(moe_ref_dispatch(&c, T, idx.data(), counts.data(), offsets.data(), row_of.data(), tok.data()), 0, "dispatch");
  std::vector<double> recv((size_t)T * k * d + 1), eout((size_t)T * k * d + 1), sout((size_t)T * d + 1);
  check(moe_ref_gather(&c, T, x, tok.data(), recv.data()), 0, "gather");
  check(moe_ref_expert_ffn(&c, T, recv.data(), offsets.data(), &w, x, eout.data(), c.num_shared ? sout.data() : nullptr,
                           2),
        0, "expert_ffn");
  std::vector<double> y((size_t)T * d + 1), y2((size_t)T * d + 1), yt(d);
  check(moe_ref_combine(&c, T, eout.data(), row_of.data(), tw.data(), c.num_shared ? sout.data() : nullptr, y.data()), 0,
        "combine");
  check(moe_ref_layer(&c, T, x, logits.data(), bias.data(), &w, nullptr, nullptr, y2.data(), 3), 0, "layer");
  for (int t = 0; t < T; ++t) {
    const void* xr = c.act_dtype == MOE_REF_BF16 ? (const void*)(xb.data() + (size_t)t * d)
                                                  : (const void*)(xf.data() + (size_t)t * d);
    check(moe_ref_dense_token(&c, xr, idx.data() + (size_t)t * k, tw.data() + (size_t)t * k, &w, yt.data()), 0,
          "dense_token");
  }
  for (size_t i = 0; i < (size_t)T * d; ++i)
    if (!(std::fabs(y[i] - y2[i]) <= 1e-9 * (1 + std::fabs(y[i])))) {
      std::printf("FAIL layer differs from the chain at %zu\n", i);
      ++fails;
      break;
    }
  std::vector<double> rl((size_t)T * E + 1);
  std::vector<float> wr((size_t)E * d);
  for (auto& v : wr) v = 0.02f * uniform();
  std::vector<uint16_t> wrb(wr.size());
  for (size_t i = 0; i < wr.size(); ++i) wrb[i] = to_bf16(wr[i]);
  const void* wrp = c.act_dtype == MOE_REF_BF16 ? (const void*)wrb.data() : (const void*)wr.data();
  check(moe_ref_router_logits(&c, T, x, wrp, rl.data()), 0, "router_logits");
}

}  // namespace

int main() {
  // E4M3 codec and row quantisation over every code and a ragged row
  for (int code = 0; code < 256; ++code) (void)moe_ref_e4m3_decode((uint8_t)code);
  const float specials[] = {0.f, -0.f, 448.f, -448.f, 1e9f, -1e9f, NAN, 1e-9f, 0.0019531f};
  for (float v : specials) (void)moe_ref_e4m3_encode(v);
  std::vector<float> rows(3 * 256);
  for (auto& v : rows) v = 10.f * uniform();
  std::vector<uint8_t> codes(rows.size());
  std::vector<float> scales(3 * 2);
  check(moe_ref_quantize_rows(3, 256, rows.data(), codes.data(), scales.data()), 0, "quantize_rows");

  // configs: sigmoid + groups + shared (bf16), softmax (f32), E4M3 weights with both activation forms
  moe_ref_config a{16, 4, 256, 128, 1, 128, 4, 2, 1, 0, 2.5, MOE_REF_BF16, MOE_REF_BF16, 0};
  moe_ref_config b{8, 2, 128, 128, 0, 0, 1, 1, 0, 1, 1.0, MOE_REF_F32, MOE_REF_F32, 0};
  moe_ref_config q{16, 4, 256, 256, 1, 256, 4, 2, 1, 0, 2.5, MOE_REF_BF16, MOE_REF_E4M3, 1};
  moe_ref_config q0 = q;
  q0.act_quant = 0;
  for (int T : {1, 5, 17}) {
    run_case(a, T);
    run_case(b, T);
    run_case(q, T);
    run_case(q0, T);
  }
  // invalid arguments return -1 and touch nothing
  moe_ref_config bad = a;
  bad.top_k = 0;
  std::vector<int32_t> idx(64);
  std::vector<double> tw(64);
  float lg[16] = {0}, bs[16] = {0};
  check(moe_ref_route(&bad, 1, lg, bs, idx.data(), tw.data()), -1, "route with top_k 0");
  check(moe_ref_route(&a, -1, lg, bs, idx.data(), tw.data()), -1, "route with T < 0");
  check(moe_ref_route(nullptr, 1, lg, bs, idx.data(), tw.data()), -1, "route without a config");
  std::printf(fails ? "oracle driver: %d failures\n" : "oracle driver: clean\n", fails);
  return fails ? 1 : 0;
}
