// Router device code, shared by the router kernel and the launch that runs
// the router next to the shared expert's gate/up pass.
#pragma once

#include "moe_kernels.h"

namespace moe {

// Exclusive prefix sum of cnt[0..E) into off[0..E] (LDS), 256 threads, E <= 1024.
__device__ inline void block_offsets(const int* cnt, int E, int* off, int* wsum) {
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

// LDS floats one routing wave needs: keys[E], scores[E], and 384 words of
// group and selection scratch.
__host__ __device__ inline int route_lds_floats(int E) { return 2 * E + 384; }

// ---------------------------------------------------------------------------
// Router: one wavefront per token.  Lane l holds experts l*KPL .. l*KPL+KPL-1.
// Selection takes k rounds of wave-wide argmax (DPP maximum of the lanes'
// best ordered keys, then the lowest lane holding it): round j picks slot j
// of the (key descending, index ascending) order directly, so the chosen
// experts need no separate sort.
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

// Largest value over the wave, in every lane: DPP row shifts combine each
// row of 16 lanes into its last lane, row broadcasts carry rows 0 and 2 into
// rows 1 and 3 and then row 1 into rows 2 and 3, so lane 63 ends with the
// maximum (lanes without a source take 0, the identity for unsigned max).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false));  // row_shr:1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false));  // row_shr:2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false));  // row_shr:4
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false));  // row_shr:8
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));  // row_bcast:15
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false));  // row_bcast:31
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Selection of token t by the calling wave, with no side effects: lane j < k
// gets the expert of slot j (slots by descending key) in my_idx and its gate
// weight (routed_scale applied) in my_w.  kbuf holds route_lds_floats(E)
// floats of this wave's LDS.  COHERENT: the logits are read with device-scope
// loads (they were written earlier in the same launch by other workgroups).
template <int KPL, bool COHERENT = false>
__device__ __forceinline__ void route_select(const RouteParams& p, int t, float* kbuf, int& my_idx, float& my_w) {
  const int lane = threadIdx.x & 63;
  const int E = p.E;
  // per-wave LDS: keys[E], scores[E], group scores[64], group chosen[64]
  float* sbuf = kbuf + E;
  float* gbuf = sbuf + E;
  float* cbuf = gbuf + 64;

  const float* lg = p.logits + (size_t)t * E;
  // every load first (past-the-end lanes read expert 0), so that they are in
  // flight together
  float lv[KPL], bv[KPL];
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const int e = lane * KPL + i < E ? lane * KPL + i : 0;
    lv[i] = COHERENT ? __hip_atomic_load(lg + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : lg[e];
  }
  const bool biased = p.score_fn == MOE_SCORE_SIGMOID && p.bias;
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const int e = lane * KPL + i < E ? lane * KPL + i : 0;
    bv[i] = biased ? p.bias[e] : 0.f;
  }
  float key[KPL];
  float lmax = -INFINITY;
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const int e = lane * KPL + i;
    float k = -INFINITY, s = 0.f;
    if (e < E) {
      const float l = lv[i];
      if (p.score_fn == MOE_SCORE_SIGMOID) {
        // sigmoid evaluated in double and rounded once to fp32
        s = (float)(1.0 / (1.0 + exp(-(double)l)));
        k = biased ? s + bv[i] : s;
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
  const int lpg = gsize / KPL;  // lanes per group when every lane's experts lie in one group
  bool elig[KPL];
  if (G > 1 && gsize % KPL == 0 && (lpg & (lpg - 1)) == 0) {
    // each group is lpg consecutive lanes: its two largest keys by a
    // butterfly of (largest, second largest) pairs inside the group, then
    // each lane ranks its group against every group's score (readlane)
    float b1 = -INFINITY, b2 = -INFINITY;
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
      const float v = key[i];
      if (v > b1) { b2 = b1; b1 = v; }
      else if (v > b2) b2 = v;
    }
    for (int off = 1; off < lpg; off <<= 1) {
      const float o1 = __shfl_xor(b1, off), o2 = __shfl_xor(b2, off);
      const float n1 = fmaxf(b1, o1);
      b2 = fmaxf(fminf(b1, o1), fmaxf(b2, o2));
      b1 = n1;
    }
    float gs = gsize == 1 ? b1 : b1 + b2;
    if (gs != gs) gs = -INFINITY;
    const int myg = lane / lpg;
    int rank = 0;
    for (int g = 0; g < G; ++g) {
      const float sg = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gs), g * lpg));
      rank += better(sg, g, gs, myg) ? 1 : 0;
    }
#pragma unroll
    for (int i = 0; i < KPL; ++i) elig[i] = lane * KPL + i < E && rank < p.topk_group;
  } else if (G > 1) {
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

  // ---- top-k: k rounds of wave-wide argmax over the eligible experts'
  // ordered keys.  Ties go to the lowest index (the lowest lane, then the
  // lowest of its experts), so round j yields slot j of the (key descending,
  // index ascending) order; the caller's configuration has at least k
  // eligible experts.
  const int k = p.k;
  uint32_t u[KPL];
#pragma unroll
  for (int i = 0; i < KPL; ++i) u[i] = elig[i] ? ord(key[i]) : 0u;  // 0: below every ordered key
  my_idx = 0;
  for (int j = 0; j < k; ++j) {
    uint32_t lb = u[0];
    int bi = 0;
#pragma unroll
    for (int i = 1; i < KPL; ++i)
      if (u[i] > lb) {
        lb = u[i];
        bi = i;
      }
    const uint32_t m = wave_max_u32(lb);
    const int L = __builtin_ctzll(__ballot(lb == m));  // lowest lane holding the maximum
    const int e = __builtin_amdgcn_readlane(lane * KPL + bi, L);
    if (lane == L) {
#pragma unroll
      for (int i = 0; i < KPL; ++i) u[i] = i == bi ? 0u : u[i];
    }
    if (lane == j) my_idx = e;
  }
  const float my_s = lane < k ? sbuf[my_idx] : 0.f;  // slot j's unbiased score, in lane j

  // ---- gate weights from the unbiased scores of the k chosen experts
  // (slot j's score in lane j, read with readlane: j is uniform), summed in
  // slot order
  auto slot_val = [](float v, int j) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), j)); };
  float w = 0.f;
  if (p.score_fn == MOE_SCORE_SOFTMAX) {
    if (p.weight_fn == MOE_WEIGHT_NORM_SUM) {
      // p_j / sum p over the chosen = exp(l_j - M) / sum exp(l_i - M); with
      // M the largest chosen logit (the largest logit overall when G = 1)
      const float m = slot_val(my_s, 0);
      float den = 0.f;
      for (int j = 0; j < k; ++j) den += expf(slot_val(my_s, j) - m);
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
      for (int j = 0; j < k; ++j) pm = fmaxf(pm, slot_val(pj, j));
      float den = 0.f;
      for (int j = 0; j < k; ++j) den += expf(slot_val(pj, j) - pm);
      w = expf(pj - pm) / den;
    }
  } else {
    if (p.weight_fn == MOE_WEIGHT_NORM_SUM) {
      float den = 0.f;
      for (int j = 0; j < k; ++j) den += slot_val(my_s, j);
      w = my_s / den;
    } else {
      float sm = -INFINITY;
      for (int j = 0; j < k; ++j) sm = fmaxf(sm, slot_val(my_s, j));
      float den = 0.f;
      for (int j = 0; j < k; ++j) den += expf(slot_val(my_s, j) - sm);
      w = expf(my_s - sm) / den;
    }
  }
  my_w = w * p.routed_scale;
}

// Routes token bid * NW + w with wave w of an NW-wave block; smem holds
// route_lds_floats(E) floats per wave.  Returns, in lane j < k, the
// masked-layout row of the token's slot j (when p.fuse; 0 otherwise), and -1
// in every lane when the token is past T.  With TICKET = false the slots take
// no ticket here (the caller reserves them) and lane j < k returns the
// expert of slot j instead.
template <int KPL, int NW, bool TICKET = true>
__device__ __forceinline__ int route_body(const RouteParams& p, int bid, float* smem) {
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int t = bid * NW + wid;
  float* kbuf = smem + wid * route_lds_floats(p.E);
  if (t >= p.T) return -1;  // uniform per wave; no block barrier is used below
  int my_idx;
  float w;
  route_select<KPL>(p, t, kbuf, my_idx, w);
  const int k = p.k;
  int my_row = 0;
  if (lane < k) {
    const size_t o = (size_t)t * k + lane;
    p.topk_idx[o] = my_idx;
    p.topk_w[o] = w;
    if constexpr (TICKET) {
      const int tk = atomicAdd(p.expert_count + my_idx, 1);
      if (p.ticket) p.ticket[o] = tk;
      if (p.fuse) {
        my_row = tk < p.T ? my_idx * p.T + tk : -1;  // -1: stale counters, the slot writes no row
        p.row_of[o] = my_row;
      }
    } else {
      my_row = my_idx;
    }
  }
  return my_row;
}

// Masked layout, one token per 256-thread workgroup: wave 0 routes it, then
// the whole workgroup writes it into the k rows its tickets reserved ("One-
// Sided Expert-Parallel All-to-All", abstract: tokens are pushed straight
// into expert-grouped buffers).  Plain rows are copied 16 bytes per thread;
// E4M3 rows are quantised per 128 columns (one block per wave, two values
// per lane) with the same arithmetic as the dispatch kernel, and also written
// to row E*T + t for the shared expert when p.shared_rows.  smem holds
// route_lds_floats(E) floats.
template <int KPL>
__device__ __forceinline__ void route_dispatch_block(const RouteParams& p, int t, float* smem) {
  __shared__ int rows_s[65];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  constexpr int NWAVE = 4;
  if (wid == 0) {
    const int my_row = route_body<KPL, 1>(p, t, smem);
    if (lane < p.k) rows_s[lane] = my_row;
    if (lane == 0) rows_s[p.k] = p.E * p.T + t;
  }
  __syncthreads();
  const int k = p.k, d = p.d;
  if (!p.quant) {
    const int eb = p.act_dtype == MOE_F32 ? 4 : 2;
    const int pieces = d * eb / 16;
    const i32x4_t* src = reinterpret_cast<const i32x4_t*>(static_cast<const uint8_t*>(p.x) + (size_t)t * d * eb);
    for (int c = tid; c < pieces; c += 64 * NWAVE) {
      const i32x4_t v = src[c];
      for (int j = 0; j < k; ++j)
        if (rows_s[j] >= 0)
          reinterpret_cast<i32x4_t*>(static_cast<uint8_t*>(p.recv) + (size_t)rows_s[j] * d * eb)[c] = v;
    }
    return;
  }
  const int nb = d / 128;
  const int nrows = p.shared_rows ? k + 1 : k;
  const uint32_t* src = reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(p.x) + (size_t)t * d);
  for (int b = wid; b < nb; b += NWAVE) {  // uniform per wave
    const uint32_t pair = src[b * 64 + lane];
    const float v0 = bf16_bits_to_f32(pair & 0xFFFFu), v1 = bf16_bits_to_f32(pair >> 16);
    float amax = fmaxf(fabsf(v0), fabsf(v1));
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    const float scale = amax > 0.f ? amax / 448.0f : 1.0f;
    const uint32_t c0 = f32_to_e4m3(v0 / scale), c1 = f32_to_e4m3(v1 / scale);
    const uint16_t codes = (uint16_t)(c0 | (c1 << 8));
    for (int j = 0; j < nrows; ++j) {
      const int r = rows_s[j];
      if (r < 0) continue;  // stale counters: the slot writes no row
      uint8_t* dst = static_cast<uint8_t*>(p.recv) + (size_t)r * d;
      reinterpret_cast<uint16_t*>(dst + b * 128)[lane] = codes;
      if (lane == 0) p.recv_scale[(size_t)r * nb + b] = scale;
    }
  }
}

}  // namespace moe
