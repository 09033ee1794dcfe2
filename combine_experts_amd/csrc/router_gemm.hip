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
#include "moe_kernels.h"

namespace moe {

namespace {

constexpr int kWaves = 4;
constexpr int kMaxTokens = 16;

// 16-byte piece -> 8 bf16 values or 4 fp32 values
template <int DT> struct Piece;
template <> struct Piece<MOE_BF16> {
  static constexpr int kElems = 8;
  static __device__ __forceinline__ float get(const i32x4_t& v, int i) {
    const uint32_t w = (uint32_t)v[i >> 1];
    return bf16_bits_to_f32((i & 1) ? (w >> 16) : (w & 0xFFFFu));
  }
};
template <> struct Piece<MOE_F32> {
  static constexpr int kElems = 4;
  static __device__ __forceinline__ float get(const i32x4_t& v, int i) { return __int_as_float(v[i]); }
};

template <int DT, int PPL>
__global__ __launch_bounds__(64 * kWaves) void router_gemv_kernel(const uint8_t* __restrict__ x,
                                                                  const uint8_t* __restrict__ w, float* logits,
                                                                  int T, int E, int d) {
  constexpr int EL = Piece<DT>::kElems;
  constexpr int ES = 16 / EL;  // bytes per element
  __shared__ float part[kWaves][kMaxTokens];
  const int e = blockIdx.x;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int pieces = d / EL;                         // 16-byte pieces per row
  const int per_wave = (pieces + kWaves - 1) / kWaves;
  const int p0 = wid * per_wave;
  const int p1 = min(pieces, p0 + per_wave);
  const size_t rowb = (size_t)d * ES;
  // this lane's pieces of the weight row, all loads issued before any use
  i32x4_t wp[PPL];
#pragma unroll
  for (int i = 0; i < PPL; ++i) {
    const int pc = p0 + lane + 64 * i;
    wp[i] = pc < p1 ? *reinterpret_cast<const i32x4_t*>(w + (size_t)e * rowb + (size_t)pc * 16)
                    : i32x4_t{0, 0, 0, 0};
  }
  float acc[kMaxTokens];
#pragma unroll
  for (int t = 0; t < kMaxTokens; ++t) acc[t] = 0.f;
#pragma unroll
  for (int t = 0; t < kMaxTokens; ++t) {
    if (t < T) {
      i32x4_t xp[PPL];
#pragma unroll
      for (int i = 0; i < PPL; ++i) {
        const int pc = p0 + lane + 64 * i;
        xp[i] = pc < p1 ? *reinterpret_cast<const i32x4_t*>(x + (size_t)t * rowb + (size_t)pc * 16)
                        : i32x4_t{0, 0, 0, 0};
      }
      float a = 0.f;
#pragma unroll
      for (int i = 0; i < PPL; ++i)
#pragma unroll
        for (int j = 0; j < EL; ++j) a = fmaf(Piece<DT>::get(xp[i], j), Piece<DT>::get(wp[i], j), a);
      acc[t] = a;
    }
  }
  // lanes -> one sum per token (fixed butterfly), waves -> LDS
#pragma unroll
  for (int t = 0; t < kMaxTokens; ++t) {
    if (t < T) {
      float a = acc[t];
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) a += __shfl_xor(a, o);
      if (lane == 0) part[wid][t] = a;
    }
  }
  __syncthreads();
  if (threadIdx.x < T) {
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < kWaves; ++q) s += part[q][threadIdx.x];
    logits[(size_t)threadIdx.x * E + e] = s;
  }
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

}  // namespace moe
