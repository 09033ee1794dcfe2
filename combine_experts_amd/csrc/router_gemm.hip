// Router GEMM for a handful of tokens: logits[t][e] = x[t] . w_router[e]
// ("7.13 Serving Mixture-of-Experts", moe_ep_layer listing: one linear map
// from the token to a score per expert, before the softmax and top-k).
//
// With T <= 16 tokens the product is a batch of dot products over a small
// weight (E x d), so it is latency-bound: what matters is spreading the
// weight over many waves with every load of a wave in flight at once.  One
// workgroup per expert; its four waves split the reduction dimension; each
// lane multiplies 16-byte pieces of the weight row by the same pieces of
// every token (fused multiply-adds in a fixed order), then the lanes reduce
// with a fixed shuffle tree and the four waves add their sums through LDS in
// wave order.  The result is reproducible run to run.
//
// The file also holds the second launch of the split router GEMM (larger
// batches, LDS-tiled kernel with its reduction in parts): the sum of the
// parts' fp32 partial sums in part order.
#include "router_gemv.h"

namespace moe {

namespace {

constexpr int kWaves = kGemvWaves;
constexpr int kMaxTokens = kGemvMaxTokens;

template <int DT, int PPL>
__global__ __launch_bounds__(64 * kWaves) void router_gemv_kernel(const uint8_t* __restrict__ x,
                                                                  const uint8_t* __restrict__ w, float* logits,
                                                                  int T, int E, int d) {
  __shared__ float part[kWaves][kMaxTokens];
  router_gemv_body<DT, PPL>(x, w, logits, T, E, d, blockIdx.x, part);
}

}  // namespace

bool router_gemv_fits(int T, int d, int dtype) {
  if (T < 1 || T > kMaxTokens || (dtype != MOE_BF16 && dtype != MOE_F32)) return false;
  const int el = dtype == MOE_BF16 ? 8 : 4;
  if (d % el) return false;
  const int per_wave = (d / el + kWaves - 1) / kWaves;
  return (per_wave + 63) / 64 <= 8;  // up to 8 pieces per lane: d <= 16384 (bf16), 8192 (fp32)
}

hipError_t launch_router_gemv(const void* x, const void* w, float* logits, int T, int E, int d, int dtype,
                              hipStream_t stream) {
  if (!router_gemv_fits(T, d, dtype) || E < 1) return hipErrorInvalidValue;
  const int el = dtype == MOE_BF16 ? 8 : 4;
  const int ppl = ((d / el + kWaves - 1) / kWaves + 63) / 64;
  const uint8_t* xb = static_cast<const uint8_t*>(x);
  const uint8_t* wb = static_cast<const uint8_t*>(w);
#define MOE_GEMV_CASE(P)                                                                                \
  if (ppl <= P) {                                                                                       \
    if (dtype == MOE_BF16)                                                                              \
      hipLaunchKernelGGL((router_gemv_kernel<MOE_BF16, P>), dim3(E), dim3(64 * kWaves), 0, stream, xb, wb, \
                         logits, T, E, d);                                                             \
    else                                                                                                \
      hipLaunchKernelGGL((router_gemv_kernel<MOE_F32, P>), dim3(E), dim3(64 * kWaves), 0, stream, xb, wb,  \
                         logits, T, E, d);                                                             \
    return hipGetLastError();                                                                           \
  }
  MOE_GEMV_CASE(1)
  MOE_GEMV_CASE(2)
  MOE_GEMV_CASE(4)
  MOE_GEMV_CASE(8)
#undef MOE_GEMV_CASE
  return hipErrorInvalidValue;
}

// The split router GEMM's partial sums -> logits: logits[i] = sum over the
// parts q = 0 .. P-1 of part[q][i], added in that order (fp32), four values
// per thread.
__global__ __launch_bounds__(256) void router_split_sum_kernel(const float* __restrict__ part, float* logits,
                                                               long long n, int P) {
  const long long i = ((long long)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  f32x4_t acc = *reinterpret_cast<const f32x4_t*>(part + i);
  for (int q = 1; q < P; ++q) {
    const f32x4_t v = *reinterpret_cast<const f32x4_t*>(part + (size_t)q * n + i);
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] += v[j];
  }
  *reinterpret_cast<f32x4_t*>(logits + i) = acc;
}

hipError_t launch_router_split_sum(const float* part, float* logits, long long n, int P, hipStream_t stream) {
  if (n <= 0 || n % 4 || P < 1) return hipErrorInvalidValue;
  const long long blocks = (n / 4 + 255) / 256;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(router_split_sum_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, part, logits, n, P);
  return hipGetLastError();
}

}  // namespace moe
