// Combine: gather each token's k expert outputs and reduce them with the gate
// weights in fp32, then add the shared expert's output.  "7.13 Serving
// Mixture-of-Experts", "Expert Parallelism Mechanics" step 4 and the
// moe_ep_layer listing (weighted scatter-add to the home token), written here
// as a gather so every output element has one writer and a fixed summation
// order (slot j = 0..k-1, then the shared term).
#include "moe_kernels.h"

namespace moe {

template <int ACT>
__global__ __launch_bounds__(256) void combine_kernel(CombineParams p) {
  // the column chunks of one token are consecutive workgroups, so the reads
  // of each expert-output row run in address order
  const int nch = (p.d / 4 + 255) / 256;
  const int t = blockIdx.x / nch;
  const int c = ((blockIdx.x - t * nch) * 256 + threadIdx.x) * 4;  // first of 4 columns
  if (blockIdx.x == 0)
    for (int e = threadIdx.x; e < p.E; e += 256) p.expert_count[e] = 0;  // ready for the next route
  if (c >= p.d) return;
  const int k = p.k;
  const int* rows = p.row_of + (size_t)t * k;
  const float* w = p.topk_w + (size_t)t * k;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  // eight slots at a time: their row indices and weights first, then all
  // eight row loads in flight together, then the FMAs in slot order
  for (int j0 = 0; j0 < k; j0 += 8) {
    int r[8];
    float wj[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      r[j] = j0 + j < k ? rows[j0 + j] : 0;
      wj[j] = j0 + j < k ? w[j0 + j] : 0.f;
      // a slot that got no row (counters left non-zero by an earlier failed
      // call) reads row 0 with weight 0
      if (r[j] < 0 || r[j] >= p.routed_rows) {
        r[j] = 0;
        wj[j] = 0.f;
      }
    }
    f32x4_t v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j0 + j < k) v[j] = *reinterpret_cast<const f32x4_t*>(p.expert_out + (size_t)r[j] * p.d + c);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j0 + j < k) {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = fmaf(wj[j], v[j][i], acc[i]);
      }
  }
  if (p.shared_out) {
    const f32x4_t s = *reinterpret_cast<const f32x4_t*>(p.shared_out + (size_t)t * p.d + c);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] += s[i];
  }
  if constexpr (ACT == MOE_F32) {
    *reinterpret_cast<f32x4_t*>(static_cast<float*>(p.y) + (size_t)t * p.d + c) = acc;
  } else {
    const uint32_t lo = f32_to_bf16_bits(acc[0]) | (f32_to_bf16_bits(acc[1]) << 16);
    const uint32_t hi = f32_to_bf16_bits(acc[2]) | (f32_to_bf16_bits(acc[3]) << 16);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.y) + (size_t)t * p.d + c) = make_uint2(lo, hi);
  }
}

hipError_t launch_combine(const CombineParams& p, hipStream_t stream) {
  const long long blocks = (long long)p.T * ((p.d / 4 + 255) / 256);
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks), block(256);
  if (p.act_dtype == MOE_F32)
    hipLaunchKernelGGL(combine_kernel<MOE_F32>, grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL(combine_kernel<MOE_BF16>, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace moe
