// Router and one-sided dispatch kernels.
//
// Router: "Mixture-of-experts serving" (learn-kernels) paragraph 1 (sigmoid
// affinity + per-expert bias that steers selection), paragraph 4
// (group-limited routing); "7.13 Serving Mixture-of-Experts", moe_ep_layer
// listing (softmax, top-k, renormalise).  Dispatch: "One-Sided
// Expert-Parallel All-to-All ... over NVLink" (abstract): tokens are pushed
// without a metadata exchange into expert-grouped buffers read in place; a
// token reserves its slot with an atomic add on its expert's counter.
#include "route_body.h"

namespace moe {

template <int KPL>
__global__ __launch_bounds__(256) void route_kernel(RouteParams p) {
  extern __shared__ float smem[];
  route_body<KPL, 4>(p, blockIdx.x, smem);
}

// Large batches: 16 tokens per workgroup, and the tickets of the workgroup's
// slots reserved with one atomic per expert.  Each slot first takes its rank
// among the workgroup's slots of its expert (an LDS atomic); then one thread
// per expert adds the workgroup's count to the expert's counter and gets the
// base.  A hot expert's counter then sees one atomic per workgroup instead of
// one per slot (4096 tokens with Zipf-skewed routing: up to 2119 slots of one
// expert).  Which ticket a slot gets within its expert is not fixed either
// way; the set of tickets is 0 .. count - 1.
constexpr int kAggWaves = 16;

template <int KPL>
__global__ __launch_bounds__(64 * kAggWaves) void route_agg_kernel(RouteParams p) {
  extern __shared__ float smem[];
  __shared__ int cnt[256], base[256];
  for (int e = threadIdx.x; e < p.E; e += 64 * kAggWaves) cnt[e] = 0;
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kAggWaves + (threadIdx.x >> 6);
  const int e = route_body<KPL, kAggWaves, false>(p, blockIdx.x, smem);
  const bool slot = t < p.T && lane < p.k;
  int rank = 0;
  if (slot) rank = atomicAdd(&cnt[e], 1);
  __syncthreads();
  for (int g = threadIdx.x; g < p.E; g += 64 * kAggWaves)
    if (cnt[g] > 0) base[g] = atomicAdd(p.expert_count + g, cnt[g]);
  __syncthreads();
  if (slot) p.ticket[(size_t)t * p.k + lane] = base[e] + rank;
}

template <int KPL>
__global__ __launch_bounds__(256) void route_dispatch_kernel(RouteParams p) {
  extern __shared__ float smem[];
  route_dispatch_block<KPL>(p, blockIdx.x, smem);
}

// Four tokens per workgroup, one per wave (256 tokens or more: sixteen, with
// tickets reserved per workgroup); with the masked-layout write (p.fuse) one
// token per workgroup, whose four waves share the copy.
hipError_t launch_route(const RouteParams& p, hipStream_t stream) {
  const int kpl_needed = (p.E + 63) / 64;
  if (!p.fuse && p.T >= 256 && p.E <= 256 && p.ticket) {  // LDS: 16 waves x (2E + 384) floats <= 57 KB
    const int blocks = (p.T + kAggWaves - 1) / kAggWaves;
    const size_t lds = kAggWaves * (size_t)route_lds_floats(p.E) * sizeof(float);
#define MOE_AGG_CASE(K)                                                                                 \
    if (kpl_needed <= K) {                                                                              \
      hipLaunchKernelGGL(route_agg_kernel<K>, dim3(blocks), dim3(64 * kAggWaves), lds, stream, p);     \
      return hipGetLastError();                                                                         \
    }
    MOE_AGG_CASE(1)
    MOE_AGG_CASE(2)
    MOE_AGG_CASE(4)
    MOE_AGG_CASE(8)
#undef MOE_AGG_CASE
  }
  const int nw = p.fuse ? 1 : 4;
  const int blocks = (p.T + nw - 1) / nw;
  const size_t lds = nw * (size_t)route_lds_floats(p.E) * sizeof(float);
#define MOE_ROUTE_CASE(K)                                                                            \
  if (kpl_needed <= K) {                                                                             \
    if (p.fuse) hipLaunchKernelGGL(route_dispatch_kernel<K>, dim3(blocks), dim3(256), lds, stream, p); \
    else hipLaunchKernelGGL(route_kernel<K>, dim3(blocks), dim3(256), lds, stream, p);               \
    return hipGetLastError();                                                                        \
  }
  MOE_ROUTE_CASE(1)
  MOE_ROUTE_CASE(2)
  MOE_ROUTE_CASE(4)
  MOE_ROUTE_CASE(8)
  MOE_ROUTE_CASE(16)
#undef MOE_ROUTE_CASE
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Dispatch: a row of blocks per token.  Every block recomputes the exclusive
// scan of the expert counters in LDS (no separate count pass), then writes
// its part of the token into the rows the token reserved.
// ---------------------------------------------------------------------------

// Grid (T, column blocks).  Compact layout: rows follow from the offsets
// scan; masked layout: row = expert * T + ticket, no scan.  Plain rows: a
// block copies 4096 bytes of its token (256 threads x 16 B); E4M3 rows: a
// block quantises eight 128-column blocks, two per wave (each half-wave
// holds one block, four values per lane).  The token's bytes
// and its slot tickets are loaded before the offsets scan so that their
// latency overlaps it.
template <int ACT, bool QUANT>
__global__ __launch_bounds__(256) void dispatch_kernel(DispatchParams p) {
  __shared__ int off[1025];
  __shared__ int wsum[4];
  __shared__ int rows[65];
  const int t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int k = p.k, d = p.d;
  int my_e = 0, my_ticket = 0;
  if (tid < k) {
    const size_t o = (size_t)t * k + tid;
    my_e = p.topk_idx[o];
    my_ticket = p.ticket[o];
  }
  constexpr int EB = Elem<ACT>::kBytes;
  // plain: this thread's 16-byte piece; E4M3: this lane's four values of
  // its half-wave's 128-column block
  const int piece = blockIdx.y * 256 + tid;
  const int pieces = d * EB / 16;
  const int nb = d / 128;
  const int blk = blockIdx.y * 8 + wid * 2 + (lane >> 5);
  const int hl = lane & 31;  // lane within the half-wave
  i32x4_t v{};
  uint2 quad{0u, 0u};
  if constexpr (!QUANT) {
    if (piece < pieces)
      v = reinterpret_cast<const i32x4_t*>(static_cast<const uint8_t*>(p.x) + (size_t)t * d * EB)[piece];
  } else {
    if (blk < nb)
      quad = reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p.x) + (size_t)t * d)[blk * 32 + hl];
  }
  if (!p.masked) {  // uniform: the scan's barriers are met by every thread
    block_offsets(p.expert_count, p.E, off, wsum);
    if (blockIdx.x == 0 && blockIdx.y == 0)
      for (int e = tid; e <= p.E; e += 256) p.expert_offset[e] = min(off[e], p.routed_rows);
  }
  if (tid < k) {
    int r = p.masked ? my_e * p.T + my_ticket : off[my_e] + my_ticket;
    // counters left non-zero by an earlier failed call: a slot whose row
    // falls outside its expert's rows or the buffer writes nothing
    if ((p.masked && my_ticket >= p.T) || r >= p.routed_rows) r = -1;
    rows[tid] = r;
    if (blockIdx.y == 0) p.row_of[(size_t)t * k + tid] = r;
  }
  if (tid == 0) rows[k] = QUANT && p.shared_rows ? p.routed_rows + t : -1;
  __syncthreads();
  const int nrows = (QUANT && p.shared_rows) ? k + 1 : k;

  if constexpr (!QUANT) {
    if (piece < pieces)
      for (int j = 0; j < nrows; ++j)
        if (rows[j] >= 0)
          reinterpret_cast<i32x4_t*>(static_cast<uint8_t*>(p.recv) + (size_t)rows[j] * d * EB)[piece] = v;
  } else {
    // the block's amax over its half-wave (both halves shuffle together; a
    // half past the last block holds zeros and stores nothing)
    const float v0 = bf16_bits_to_f32(quad.x & 0xFFFFu), v1 = bf16_bits_to_f32(quad.x >> 16);
    const float v2 = bf16_bits_to_f32(quad.y & 0xFFFFu), v3 = bf16_bits_to_f32(quad.y >> 16);
    float amax = fmaxf(fmaxf(fabsf(v0), fabsf(v1)), fmaxf(fabsf(v2), fabsf(v3)));
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    if (blk < nb) {
      const float scale = amax > 0.f ? amax / 448.0f : 1.0f;
      const uint32_t codes = f32_to_e4m3(v0 / scale) | (f32_to_e4m3(v1 / scale) << 8) |
                             (f32_to_e4m3(v2 / scale) << 16) | (f32_to_e4m3(v3 / scale) << 24);
      for (int j = 0; j < nrows; ++j) {
        if (rows[j] < 0) continue;
        uint8_t* dst = static_cast<uint8_t*>(p.recv) + (size_t)rows[j] * d;
        reinterpret_cast<uint32_t*>(dst + blk * 128)[hl] = codes;
        if (hl == 0) p.recv_scale[(size_t)rows[j] * nb + blk] = scale;
      }
    }
  }
}

hipError_t launch_dispatch(const DispatchParams& p, hipStream_t stream) {
  const dim3 block(256);
  if (p.quant) {
    const dim3 grid(p.T, (p.d / 128 + 7) / 8);
    hipLaunchKernelGGL((dispatch_kernel<MOE_BF16, true>), grid, block, 0, stream, p);
  } else if (p.act_dtype == MOE_F32) {
    const dim3 grid(p.T, (p.d * 4 / 16 + 255) / 256);
    hipLaunchKernelGGL((dispatch_kernel<MOE_F32, false>), grid, block, 0, stream, p);
  } else {
    const dim3 grid(p.T, (p.d * 2 / 16 + 255) / 256);
    hipLaunchKernelGGL((dispatch_kernel<MOE_BF16, false>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace moe
