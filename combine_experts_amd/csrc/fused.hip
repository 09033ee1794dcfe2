// The whole MoE layer for a handful of tokens in one persistent launch: the
// single-GPU form of the fused MoE kernel that "DeepSeek MoE Serving: Where
// Expert-Parallel All-to-All Time Goes" (section "The batch-scaling curve is
// the diagnostic") describes, which runs dispatch, both expert GEMMs and
// combine in one kernel.  "7.13 Serving Mixture-of-Experts", section
// "DeepEP", trick 3: at decode batch sizes the per-layer launch overhead can
// rival the work itself.
//
// Design (gfx950), one 256-thread workgroup per CU, all of them resident:
//  1. (optional) router GEMM: logits = x W_r^T, the experts spread over the
//     grid with the router kernel's dot-product code; a grid barrier.
//  2. Routing, by every workgroup on its own: the T <= 16 tokens are routed
//     in LDS with the router kernel's selection code (one wave per token),
//     and the canonical dispatch layout (an expert's rows in ascending token
//     order) is derived from the choices.  Every workgroup derives the same
//     layout, so no counter, ticket or exchange is needed, and dispatch
//     needs no copy: the gate/up pass reads each row straight from its token.
//  3. gate/up + SwiGLU over all touched experts and the shared expert (the
//     weight-streaming walk of the decode GEMM kernel); a grid barrier.
//  4. down pass (same walk); a grid barrier.
//  5. combine: y[t] = sum_j w[t][j] out[row(t, j)] + shared[t], fp32 in slot
//     order, rounded once.
// A grid barrier is an agent-scope release (the workgroup's stores reach
// device coherence), an atomic arrival count and a bounded wait for the full
// count, then an agent-scope acquire, once per workgroup.  The last workgroup to finish zeroes the
// counters, so the workspace is ready for the next call.  A wait that runs
// past its bound sets the error word and lets the workgroup go on, so every
// wave always reaches the end of the kernel.
#include "ffn_body.h"
#include "router_gemv.h"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxT = 16;
constexpr int kMaxSlots = 256;  // T * k
constexpr int kMaxE = 256;
constexpr int kKpl = kMaxE / 64;

// Grid-wide barrier.  Every wave first waits until its own stores have
// reached its XCD's L2 (s_waitcnt vmcnt(0)); then one thread per workgroup
// makes them visible to the other XCDs (agent-scope release: one L2
// write-back), counts itself in, waits for the full count, and invalidates
// its CU's L1 and its XCD's L2 lines (agent-scope acquire) before the
// workgroup goes on.  Cache maintenance once per workgroup rather than once
// per wave: measured on 256 workgroups, 26.8 us per barrier with a release
// and an acquire in every wave.
__device__ __forceinline__ void grid_barrier(int* ctr, int nblk, int* err, int spin_limit) {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's stores are done
  __syncthreads();
  if (threadIdx.x == 0) {
    __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    int n = 0;
    while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < nblk) {
      __builtin_amdgcn_s_sleep(2);
      if (++n >= spin_limit) {
        __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
}

template <int PPL>
__device__ __forceinline__ void router_phase(const FusedParams& fp, int bid, int nblk,
                                             float (*part)[kGemvMaxTokens]) {
  const int E = fp.r.E;
  for (int e = bid; e < E; e += nblk) {
    router_gemv_body<MOE_BF16, PPL>(static_cast<const uint8_t*>(fp.x), static_cast<const uint8_t*>(fp.w_router),
                                    fp.logits_ws, fp.r.T, E, fp.d, e, part);
    __syncthreads();  // part is reused by the next expert
  }
}

}  // namespace

template <int AFW, int AKS, bool ASH, int BFW, int BKS, bool BSH>
__global__ __launch_bounds__(kThreads) void fused_layer_kernel(FusedParams fp) {
  extern __shared__ float route_smem[];  // four waves x route_lds_floats(E)
  __shared__ int s_idx[kMaxSlots];
  __shared__ float s_w[kMaxSlots];
  __shared__ int s_row[kMaxSlots];  // compact row of slot (t, j)
  __shared__ int s_tok[kMaxSlots];  // token of compact row r
  __shared__ int s_cnt[kMaxE];
  __shared__ int s_off[kMaxE + 1];
  __shared__ int s_wsum[4];
  __shared__ float s_part[kGemvWaves][kGemvMaxTokens];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int bid = blockIdx.x, nblk = gridDim.x;
  const int T = fp.r.T, E = fp.r.E, k = fp.r.k;

  // ---- 1. router GEMM (when the logits are not an input)
  if (fp.w_router) {
    const int ppl = ((fp.d / 8 + kGemvWaves - 1) / kGemvWaves + 63) / 64;
    if (ppl <= 1) router_phase<1>(fp, bid, nblk, s_part);
    else if (ppl <= 2) router_phase<2>(fp, bid, nblk, s_part);
    else if (ppl <= 4) router_phase<4>(fp, bid, nblk, s_part);
    else router_phase<8>(fp, bid, nblk, s_part);
    grid_barrier(fp.sync + 0, nblk, fp.err, fp.spin_limit);
  }

  // ---- 2. routing of every token by this workgroup, canonical layout in LDS
  for (int t = wid; t < T; t += kThreads / 64) {  // uniform per wave
    int my_idx;
    float my_w;
    route_select<kKpl>(fp.r, t, route_smem + wid * route_lds_floats(E), my_idx, my_w);
    if (lane < k) {
      s_idx[t * k + lane] = my_idx;
      s_w[t * k + lane] = my_w;
    }
  }
  for (int e = tid; e < E; e += kThreads) s_cnt[e] = 0;
  __syncthreads();
  // slot (t, j) takes rank = number of earlier tokens that chose the same
  // expert (a token chooses an expert at most once)
  const int slots = T * k;
  int my_e = 0, my_rank = 0;
  if (tid < slots) {
    my_e = s_idx[tid];
    for (int i = 0; i < (tid / k) * k; ++i) my_rank += s_idx[i] == my_e ? 1 : 0;
    atomicAdd(&s_cnt[my_e], 1);  // LDS; the counts do not depend on the order
  }
  __syncthreads();
  block_offsets(s_cnt, E, s_off, s_wsum);
  if (tid < slots) {
    const int r = s_off[my_e] + my_rank;
    s_row[tid] = r;
    s_tok[r] = tid / k;
  }
  __syncthreads();

  // ---- 3. gate/up + SwiGLU, rows read from their tokens
  ffn_body<MOE_BF16, AFW, AKS, 1, true, MOE_BF16, 2, true, ASH, true>(fp.a, bid, nblk, s_off, s_tok);
  grid_barrier(fp.sync + 1, nblk, fp.err, fp.spin_limit);

  // ---- 4. down
  ffn_body<MOE_BF16, BFW, BKS, 1, false, MOE_F32, 2, true, BSH, true>(fp.b, bid, nblk, s_off, nullptr);
  grid_barrier(fp.sync + 2, nblk, fp.err, fp.spin_limit);

  // ---- 5. combine, in the combine kernel's arithmetic: fp32 FMAs in slot
  // order, then the shared term, one rounding to bf16
  const int d = fp.d, nch = (d + 4 * kThreads - 1) / (4 * kThreads);
  for (int item = bid; item < T * nch; item += nblk) {
    const int t = item / nch;
    const int c = ((item - t * nch) * kThreads + tid) * 4;
    if (c < d) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
      for (int j = 0; j < k; ++j) {
        const float wj = s_w[t * k + j];
        const f32x4_t v = *reinterpret_cast<const f32x4_t*>(fp.expert_out + (size_t)s_row[t * k + j] * d + c);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = fmaf(wj, v[i], acc[i]);
      }
      if (fp.shared_out) {
        const f32x4_t sv = *reinterpret_cast<const f32x4_t*>(fp.shared_out + (size_t)t * d + c);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] += sv[i];
      }
      const uint32_t lo = f32_to_bf16_bits(acc[0]) | (f32_to_bf16_bits(acc[1]) << 16);
      const uint32_t hi = f32_to_bf16_bits(acc[2]) | (f32_to_bf16_bits(acc[3]) << 16);
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(fp.y) + (size_t)t * d + c) = make_uint2(lo, hi);
    }
  }

  // ---- exit: the last workgroup out zeroes the counters for the next call
  __syncthreads();
  if (tid == 0) {
    const int done = __hip_atomic_fetch_add(fp.sync + 3, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    if (done == nblk - 1)
      for (int i = 0; i < 4; ++i) __hip_atomic_store(fp.sync + i, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

namespace {

template <int AFW, int AKS, bool ASH, int BFW, int BKS, bool BSH>
hipError_t launch_fused_shape(const FusedParams& p, hipStream_t stream) {
  auto kern = fused_layer_kernel<AFW, AKS, ASH, BFW, BKS, BSH>;
  const size_t lds = (size_t)(kThreads / 64) * route_lds_floats(kMaxE) * sizeof(float);
  // every workgroup must be resident at once (grid barriers): one per CU,
  // launched only where the occupancy calculation allows at least one, and
  // constant per kernel and device model (computed once)
  static const Residency occ = [&] {
    Residency o{};
    int dev = 0, n = 0, c = 0;
    if (hipGetDevice(&dev) != hipSuccess) return o;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, kThreads, lds) != hipSuccess) return o;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return o;
    o.per_cu = n;
    o.cus = c;
    o.ok = n >= 1 && c >= 1;
    return o;
  }();
  if (!occ.ok) return hipErrorInvalidDevice;
  hipLaunchKernelGGL(kern, dim3(occ.cus), dim3(kThreads), lds, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fused(const FusedParams& p, const FusedPlan& a, const FusedPlan& b, hipStream_t stream) {
  if (p.r.T < 1 || p.r.T > kMaxT || p.r.T * p.r.k > kMaxSlots || p.r.E > kMaxE) return hipErrorInvalidValue;
#define MOE_FUSED_B(AFW, AKS, ASH)                                                              \
  if (b.fw == 1 && b.ks == 4 && !b.share) return launch_fused_shape<AFW, AKS, ASH, 1, 4, false>(p, stream); \
  if (b.fw == 2 && b.ks == 2 && b.share) return launch_fused_shape<AFW, AKS, ASH, 2, 2, true>(p, stream);   \
  if (b.fw == 4 && b.ks == 1 && !b.share) return launch_fused_shape<AFW, AKS, ASH, 4, 1, false>(p, stream); \
  return hipErrorInvalidValue;
  if (a.fw == 1 && a.ks == 4 && !a.share) { MOE_FUSED_B(1, 4, false) }
  if (a.fw == 2 && a.ks == 2 && a.share) { MOE_FUSED_B(2, 2, true) }
  if (a.fw == 4 && a.ks == 1 && !a.share) { MOE_FUSED_B(4, 1, false) }
#undef MOE_FUSED_B
  return hipErrorInvalidValue;
}

}  // namespace moe
