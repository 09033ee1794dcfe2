// Router and one-sided dispatch kernels.
//
// Router: "Mixture-of-experts serving" (learn-kernels) paragraph 1 (sigmoid
// affinity + per-expert bias that steers selection), paragraph 4
// (group-limited routing); "7.13 Serving Mixture-of-Experts", moe_ep_layer
// listing (softmax, top-k, renormalise).  Dispatch: "One-Sided
// Expert-Parallel All-to-All ... over NVLink" (abstract): tokens are pushed
// without a metadata exchange into expert-grouped buffers read in place; a
// token reserves its slot with an atomic add on its expert's counter.
#include "moe_kernels.h"

namespace moe {

// ---------------------------------------------------------------------------
// Router: one wavefront per token.  Lane l holds experts l*KPL .. l*KPL+KPL-1.
// Selection is a radix select on wave ballots (no cross-lane shuffles): the
// k-th largest selection key is found bit by bit from the top, the experts
// above it are taken, and ties at it go to the lowest indices.  The chosen k
// are then put in (key descending, index ascending) order through LDS.
// ---------------------------------------------------------------------------

// Total order of candidates: larger key first, then lower index.
__device__ __forceinline__ bool better(float ka, int ia, float kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}

// Monotone map of a non-NaN float onto uint32 (a < b <=> ord(a) < ord(b)).
__device__ __forceinline__ uint32_t ord(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int popc64(unsigned long long m) { return __popcll(m); }

template <int KPL>
__global__ __launch_bounds__(256) void route_kernel(RouteParams p) {
  extern __shared__ float smem[];
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wid;
  const int E = p.E;
  // per-wave LDS: keys[E], scores[E], group scores[64], group chosen[64],
  // chosen (key, index) in index order [64 + 64], chosen (index, score) in
  // output order [64 + 64]
  float* kbuf = smem + wid * (2 * E + 384);
  float* sbuf = kbuf + E;
  float* gbuf = sbuf + E;
  float* cbuf = gbuf + 64;
  uint32_t* cu = reinterpret_cast<uint32_t*>(cbuf + 64);
  int* ce = reinterpret_cast<int*>(cu + 64);
  int* oe = ce + 64;
  float* os = reinterpret_cast<float*>(oe + 64);
  if (t >= p.T) return;  // uniform per wave; no block barrier is used below

  const float* lg = p.logits + (size_t)t * E;
  float key[KPL];
  float lmax = -INFINITY;
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const int e = lane * KPL + i;
    float k = -INFINITY, s = 0.f;
    if (e < E) {
      const float l = lg[e];
      if (p.score_fn == MOE_SCORE_SIGMOID) {
        // sigmoid evaluated in double and rounded once to fp32
        s = (float)(1.0 / (1.0 + exp(-(double)l)));
        k = p.bias ? s + p.bias[e] : s;
      } else {
        s = l;
        k = l;
        if (l == l) lmax = fmaxf(lmax, l);
      }
      if (k != k) k = -INFINITY;
      if (k == 0.f) k = 0.f;  // -0 and +0 compare equal: one ordered value
      kbuf[e] = k;
      sbuf[e] = s;
    }
    key[i] = k;
  }

  // ---- group stage: each group's score is the sum of its two largest keys;
  // the topk_group best groups survive
  const int G = p.n_group;
  const int gsize = E / G;
  bool elig[KPL];
  if (G > 1) {
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    // LPG lanes (a power of two) scan one group together, then merge their
    // (largest, second largest) pairs with butterflies inside the group
    int lpg = 1;
    while (lpg * 2 * G <= 64) lpg *= 2;
    const int q = lane / lpg, r = lane % lpg;
    float b1 = -INFINITY, b2 = -INFINITY;
    if (q < G) {
      for (int j = r; j < gsize; j += lpg) {
        const float v = kbuf[q * gsize + j];
        if (v > b1) { b2 = b1; b1 = v; }
        else if (v > b2) b2 = v;
      }
    }
    for (int off = 1; off < lpg; off <<= 1) {
      const float o1 = __shfl_xor(b1, off), o2 = __shfl_xor(b2, off);
      const float n1 = fmaxf(b1, o1);
      b2 = fmaxf(fminf(b1, o1), fmaxf(b2, o2));
      b1 = n1;
    }
    if (q < G && r == 0) {
      float gs = gsize == 1 ? b1 : b1 + b2;
      if (gs != gs) gs = -INFINITY;
      gbuf[q] = gs;
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    if (lane < G) {
      const float mine = gbuf[lane];
      int rank = 0;
      for (int g = 0; g < G; ++g) rank += better(gbuf[g], g, mine, lane) ? 1 : 0;
      cbuf[lane] = rank < p.topk_group ? 1.f : 0.f;
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
      const int e = lane * KPL + i;
      elig[i] = e < E && cbuf[e / gsize] != 0.f;
    }
  } else {
#pragma unroll
    for (int i = 0; i < KPL; ++i) elig[i] = lane * KPL + i < E;
  }

  // ---- top-k: u_t = the k-th largest ordered key among eligible experts,
  // found bit by bit (count(u >= t) >= k holds for the largest such t)
  const int k = p.k;
  uint32_t u[KPL];
#pragma unroll
  for (int i = 0; i < KPL; ++i) u[i] = ord(key[i]);
  uint32_t thr = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t c = thr | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < KPL; ++i) cnt += popc64(__ballot(elig[i] && u[i] >= c));
    if (cnt >= k) thr = c;
  }
  // everything above the threshold is taken; ties at it by lowest index
  const unsigned long long below = (1ull << lane) - 1ull;  // lanes with lower experts
  int n_gt = 0, tie_before = 0;
  bool gt[KPL], eq[KPL];
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    gt[i] = elig[i] && u[i] > thr;
    eq[i] = elig[i] && u[i] == thr;
    n_gt += popc64(__ballot(gt[i]));
    tie_before += popc64(__ballot(eq[i]) & below);
  }
  const int need = k - n_gt;  // >= 1
  bool sel[KPL];
  int sel_before = 0;
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    sel[i] = gt[i] || (eq[i] && tie_before < need);
    tie_before += eq[i] ? 1 : 0;
  }
#pragma unroll
  for (int i = 0; i < KPL; ++i) sel_before += popc64(__ballot(sel[i]) & below);
  // chosen experts in index order -> LDS
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    if (sel[i]) {
      cu[sel_before] = u[i];
      ce[sel_before] = lane * KPL + i;
      ++sel_before;
    }
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  // lane j < k places chosen expert j at its rank in (key desc, index asc)
  if (lane < k) {
    const uint32_t uj = cu[lane];
    const int ej = ce[lane];
    int pos = 0;
    for (int j = 0; j < k; ++j) {
      const uint32_t uo = cu[j];
      pos += (uo > uj || (uo == uj && ce[j] < ej)) ? 1 : 0;
    }
    oe[pos] = ej;
    os[pos] = sbuf[ej];
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  int my_idx = 0;
  float my_s = 0.f;
  if (lane < k) {
    my_idx = oe[lane];
    my_s = os[lane];
  }

  // ---- gate weights from the unbiased scores of the k chosen experts
  float w = 0.f;
  if (p.score_fn == MOE_SCORE_SOFTMAX) {
    if (p.weight_fn == MOE_WEIGHT_NORM_SUM) {
      // p_j / sum p over the chosen = exp(l_j - M) / sum exp(l_i - M); with
      // M the largest chosen logit (the largest logit overall when G = 1)
      const float m = os[0];
      float den = 0.f;
      for (int j = 0; j < k; ++j) den += expf(os[j] - m);
      w = expf(my_s - m) / den;
    } else {
      // p_e = exp(l_e - M) / Z over all experts
      float m = lmax;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
      float z = 0.f;
#pragma unroll
      for (int i = 0; i < KPL; ++i) {
        const int e = lane * KPL + i;
        if (e < E) z += expf(sbuf[e] - m);
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) z += __shfl_xor(z, off);
      const float pj = expf(my_s - m) / z;
      float pm = -INFINITY;
      for (int j = 0; j < k; ++j) pm = fmaxf(pm, __shfl(pj, j));
      float den = 0.f;
      for (int j = 0; j < k; ++j) den += expf(__shfl(pj, j) - pm);
      w = expf(pj - pm) / den;
    }
  } else {
    if (p.weight_fn == MOE_WEIGHT_NORM_SUM) {
      float den = 0.f;
      for (int j = 0; j < k; ++j) den += os[j];
      w = my_s / den;
    } else {
      float sm = -INFINITY;
      for (int j = 0; j < k; ++j) sm = fmaxf(sm, os[j]);
      float den = 0.f;
      for (int j = 0; j < k; ++j) den += expf(os[j] - sm);
      w = expf(my_s - sm) / den;
    }
  }
  w *= p.routed_scale;

  if (lane < k) {
    const size_t o = (size_t)t * k + lane;
    p.topk_idx[o] = my_idx;
    p.topk_w[o] = w;
    p.ticket[o] = atomicAdd(p.expert_count + my_idx, 1);
  }
}

hipError_t launch_route(const RouteParams& p, hipStream_t stream) {
  const int kpl_needed = (p.E + 63) / 64;
  const int blocks = (p.T + 3) / 4;
  const size_t lds = 4 * (2 * (size_t)p.E + 384) * sizeof(float);
#define MOE_ROUTE_CASE(K)                                                                \
  if (kpl_needed <= K) {                                                                 \
    hipLaunchKernelGGL(route_kernel<K>, dim3(blocks), dim3(256), lds, stream, p);        \
    return hipGetLastError();                                                            \
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

// Exclusive prefix sum of cnt[0..E) into off[0..E] (LDS), 256 threads, E <= 1024.
__device__ void block_offsets(const int* cnt, int E, int* off, int* wsum) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  int v[4];
  int local = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = tid * 4 + i;
    v[i] = e < E ? cnt[e] : 0;
    local += v[i];
  }
  // inclusive scan of `local` across the wave
  int inc = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(inc, o);
    if (lane >= o) inc += y;
  }
  if (lane == 63) wsum[wid] = inc;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wid; ++w) base += wsum[w];
  int run = base + inc - local;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = tid * 4 + i;
    if (e < E) off[e] = run;
    run += v[i];
  }
  if (tid == 255) off[E] = run;  // E <= 1024 = 256 * 4, so thread 255 ends the scan
  __syncthreads();
}

// Grid (T, column blocks).  Plain rows: a block copies 4096 bytes of its
// token (256 threads x 16 B); E4M3 rows: a block quantises four 128-column
// blocks (one per wave).  The token's bytes and its slot tickets are loaded
// before the offsets scan so that their latency overlaps it.
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
  // plain: this thread's 16-byte piece; E4M3: this lane's two values of the
  // wave's 128-column block
  const int piece = blockIdx.y * 256 + tid;
  const int pieces = d * EB / 16;
  const int nb = d / 128;
  const int blk = blockIdx.y * 4 + wid;
  i32x4_t v{};
  uint32_t pair = 0;
  if constexpr (!QUANT) {
    if (piece < pieces)
      v = reinterpret_cast<const i32x4_t*>(static_cast<const uint8_t*>(p.x) + (size_t)t * d * EB)[piece];
  } else {
    if (blk < nb)
      pair = reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(p.x) + (size_t)t * d)[blk * 64 + lane];
  }
  block_offsets(p.expert_count, p.E, off, wsum);
  if (blockIdx.x == 0 && blockIdx.y == 0)
    for (int e = tid; e <= p.E; e += 256) p.expert_offset[e] = off[e];
  if (tid < k) {
    const int r = off[my_e] + my_ticket;
    rows[tid] = r;
    if (blockIdx.y == 0) p.row_of[(size_t)t * k + tid] = r;
  }
  if (tid == 0) rows[k] = QUANT && p.shared_rows ? k * p.T + t : -1;
  __syncthreads();
  const int nrows = (QUANT && p.shared_rows) ? k + 1 : k;

  if constexpr (!QUANT) {
    if (piece < pieces)
      for (int j = 0; j < nrows; ++j)
        reinterpret_cast<i32x4_t*>(static_cast<uint8_t*>(p.recv) + (size_t)rows[j] * d * EB)[piece] = v;
  } else {
    if (blk < nb) {  // uniform per wave
      const float v0 = bf16_bits_to_f32(pair & 0xFFFFu), v1 = bf16_bits_to_f32(pair >> 16);
      float amax = fmaxf(fabsf(v0), fabsf(v1));
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
      const float scale = amax > 0.f ? amax / 448.0f : 1.0f;
      const uint32_t c0 = f32_to_e4m3(v0 / scale), c1 = f32_to_e4m3(v1 / scale);
      const uint16_t codes = (uint16_t)(c0 | (c1 << 8));
      for (int j = 0; j < nrows; ++j) {
        uint8_t* dst = static_cast<uint8_t*>(p.recv) + (size_t)rows[j] * d;
        reinterpret_cast<uint16_t*>(dst + blk * 128)[lane] = codes;
        if (lane == 0) p.recv_scale[(size_t)rows[j] * nb + blk] = scale;
      }
    }
  }
}

hipError_t launch_dispatch(const DispatchParams& p, hipStream_t stream) {
  const dim3 block(256);
  if (p.quant) {
    const dim3 grid(p.T, (p.d / 128 + 3) / 4);
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
