// Router dot products for a handful of tokens (device code), shared by the
// router GEMM kernel and the fused decode layer; design notes in
// router_gemm.hip.
#pragma once

#include "moe_kernels.h"

namespace moe {

constexpr int kGemvWaves = 4;
constexpr int kGemvMaxTokens = 16;

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

// Logits of expert e for all T tokens, by the calling workgroup (waves 0-3
// split d; any further waves hold no pieces and only meet the barrier); part
// holds one row of kGemvMaxTokens floats of LDS per wave.  COHERENT: the
// logits are stored with device-scope stores, for readers elsewhere in the
// same launch.
template <int DT, int PPL, bool COHERENT = false>
__device__ __forceinline__ void router_gemv_body(const uint8_t* __restrict__ x, const uint8_t* __restrict__ w,
                                                 float* logits, int T, int E, int d, int e,
                                                 float (*part)[kGemvMaxTokens]) {
  constexpr int EL = Piece<DT>::kElems;
  constexpr int ES = 16 / EL;  // bytes per element
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int pieces = d / EL;                         // 16-byte pieces per row
  const int per_wave = (pieces + kGemvWaves - 1) / kGemvWaves;
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
  float acc[kGemvMaxTokens];
#pragma unroll
  for (int t = 0; t < kGemvMaxTokens; ++t) acc[t] = 0.f;
#pragma unroll
  for (int t = 0; t < kGemvMaxTokens; ++t) {
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
  for (int t = 0; t < kGemvMaxTokens; ++t) {
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
    for (int q = 0; q < kGemvWaves; ++q) s += part[q][threadIdx.x];
    if constexpr (COHERENT)
      __hip_atomic_store(logits + (size_t)threadIdx.x * E + e, s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
      logits[(size_t)threadIdx.x * E + e] = s;
  }
}

}  // namespace moe
