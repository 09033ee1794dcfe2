// The whole MoE layer for a handful of tokens in one persistent launch: the
// single-GPU form of the fused MoE kernel that "DeepSeek MoE Serving: Where
// Expert-Parallel All-to-All Time Goes" (section "The batch-scaling curve is
// the diagnostic") describes, which runs dispatch, both expert GEMMs and
// combine in one kernel.  "7.13 Serving Mixture-of-Experts", section
// "DeepEP", trick 3: at decode batch sizes the per-layer launch overhead can
// rival the work itself.
//
// Design (gfx950), one workgroup per CU, all of them resident, five waves
// each: four streaming waves and one epilogue wave.
//  0. (optional) router GEMM: logits = x W_r^T, one expert per workgroup with
//     the router kernel's dot-product code; a grid barrier.
//  1. Routing, by every workgroup on its own: the T <= 16 tokens are routed
//     in LDS with the router kernel's selection code, and the touched experts
//     are listed in index order.  Every workgroup derives the same lists, so
//     no counter, ticket or exchange is needed, and there is no dispatch
//     copy: the gate/up pass reads the tokens themselves.
//  2. gate/up + SwiGLU.  A unit is 8 columns of one expert's h: their 8 gate
//     rows and 8 up rows of W13 form one 16-row MFMA tile (gate rows 0-7, up
//     rows 8-15) against the tokens as columns.  The units of all touched
//     experts and of the shared expert are split evenly over the grid; the
//     four streaming waves split each unit's K, and the epilogue wave adds
//     their partial sums, applies SwiGLU and writes h.
//  3. One grid barrier.
//  4. down + combine.  Each workgroup owns a slice of y's columns (the model
//     dimension, in groups of 4) for all tokens and runs every touched expert
//     and the shared expert over it, folding each expert's fp32 output into
//     the running sum with the token's gate weight (fmaf, as the combine
//     kernel does).  So the combine needs no second barrier and no expert
//     output buffer.  The streaming waves split the slice's (expert, tile,
//     K-step) sequence evenly; the epilogue wave adds their sums and writes y.
//
// Streaming: each streaming wave runs a ring of D stages in LDS.  A stage is
// one 256-byte K-step of a 16-row weight tile (4 KB) and of the token tile
// (16 bytes per lane group and token column), brought in by direct-to-LDS
// loads (global_load_lds_dwordx4), so D stages per wave are in flight without
// staging registers.  Before a stage is read the wave waits (s_waitcnt) until
// only the loads issued after the stage's own are outstanding; the streaming
// waves issue no other vector-memory operation inside their loops (no stores,
// no scratch), so the count is exact.
//
// Handoff between workgroups: h (and the router's logits) are written with
// device-scope stores and read with device-scope loads, so a grid barrier
// needs no cache write-back or invalidate: each wave waits until its own
// stores are done, then the epilogue wave counts the workgroup in and waits
// for the full count.  The wait is bounded by spin_limit; when it gives up it
// sets the error word and lets the workgroup go on, so every wave always
// reaches the end of the kernel.  The last workgroup out zeroes the counters
// for the next call.
#include "route_body.h"
#include "router_gemv.h"

namespace moe {

namespace {

constexpr int kStream = 4;     // streaming waves
constexpr int kEpi = kStream;  // index of the epilogue wave
constexpr int kWaves = kStream + 1;
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxT = 16;
constexpr int kMaxSlots = 256;
constexpr int kMaxE = 256;
constexpr int kKpl = kMaxE / 64;
constexpr int kMaxTiles = 2;  // 16-row tiles of y columns per workgroup
constexpr int kAWin = 4096;   // one stage's weight tile per wave: 16 rows x 256 bytes
constexpr int kSc1 = 16;      // cache-policy bits of a device-scope access

typedef __attribute__((address_space(3))) void lds_void;

template <int AUX>
__device__ __forceinline__ void dma16(const uint8_t* g, uint8_t* window) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)window, 16, 0, AUX);
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// One ring stage -> MFMA operands: wait until at most M of this wave's
// vector-memory operations are in flight (the loads of the stages issued
// after this one), read the stage's four weight pieces (wa, 1 KB apart) and
// four token pieces (wb[q]), and wait for the reads.  One asm block, so the
// compiler neither adds a wait of its own (it cannot tell which ring slot a
// direct-to-LDS load writes) nor sees the outputs before the reads are done.
#define MOE_STAGE_READ(M)                                                                       \
  asm volatile("s_waitcnt vmcnt(" #M ")\n\t"                                                   \
               "ds_read_b128 %0, %8\n\t"                                                       \
               "ds_read_b128 %1, %8 offset:1024\n\t"                                           \
               "ds_read_b128 %2, %8 offset:2048\n\t"                                           \
               "ds_read_b128 %3, %8 offset:3072\n\t"                                           \
               "ds_read_b128 %4, %9\n\t"                                                       \
               "ds_read_b128 %5, %10\n\t"                                                      \
               "ds_read_b128 %6, %11\n\t"                                                      \
               "ds_read_b128 %7, %12\n\t"                                                      \
               "s_waitcnt lgkmcnt(0)"                                                           \
               : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3]), "=&v"(b[0]), "=&v"(b[1]),     \
                 "=&v"(b[2]), "=&v"(b[3])                                                       \
               : "v"(wa), "v"(wb0), "v"(wb0 + bwin), "v"(wb0 + 2 * bwin), "v"(wb0 + 3 * bwin)   \
               : "memory")

// m: stages issued after this one (at most 7; 8 loads each)
__device__ __forceinline__ void stage_read(int m, uint32_t wa, uint32_t wb0, uint32_t bwin, i32x4_t (&a)[4],
                                           i32x4_t (&b)[4]) {
  switch (m) {
    case 0: MOE_STAGE_READ(0); break;
    case 1: MOE_STAGE_READ(8); break;
    case 2: MOE_STAGE_READ(16); break;
    case 3: MOE_STAGE_READ(24); break;
    case 4: MOE_STAGE_READ(32); break;
    case 5: MOE_STAGE_READ(40); break;
    case 6: MOE_STAGE_READ(48); break;
    default: MOE_STAGE_READ(56); break;
  }
}
#undef MOE_STAGE_READ

// LDS address of a shared-memory pointer
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Workgroup barrier that orders LDS only (a fence would wait for every load
// in flight); the memory clobber keeps the compiler from moving accesses
// across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Grid-wide barrier of the resident workgroups.  Every wave first waits until
// its own (device-scope) stores are done; the epilogue wave's first lane then
// counts the workgroup in and waits for the full count.
__device__ __forceinline__ void grid_sync(int* ctr, int nblk, int* err, int spin_limit) {
  wait_vm<0>();
  lds_barrier();
  if (threadIdx.x == 64 * kEpi) {
    __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int n = 0;
    while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < nblk) {
      __builtin_amdgcn_s_sleep(1);
      if (++n >= spin_limit) {
        __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
  }
  lds_barrier();
}

__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ uint32_t mix(uint32_t v) { return (v * 2654435761u) >> 16; }

template <int PPL>
__device__ __forceinline__ void router_dots(const FusedParams& fp, int e, float (*part)[kGemvMaxTokens]) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int T = fp.r.T, E = fp.r.E, d = fp.d;
  const int pieces = d / 8;
  const int per_wave = (pieces + kGemvWaves - 1) / kGemvWaves;
  const int p0 = wid * per_wave;
  const int p1 = min(pieces, p0 + per_wave);
  const uint8_t* w = reinterpret_cast<const uint8_t*>(fp.w_router) + (size_t)e * d * 2;
  const uint8_t* x = reinterpret_cast<const uint8_t*>(fp.x);
  i32x4_t wp[PPL];
#pragma unroll
  for (int i = 0; i < PPL; ++i) {
    const int pc = p0 + lane + 64 * i;
    wp[i] = pc < p1 ? *reinterpret_cast<const i32x4_t*>(w + (size_t)pc * 16) : i32x4_t{0, 0, 0, 0};
  }
#pragma unroll 1
  for (int t = 0; t < T; ++t) {
    i32x4_t xp[PPL];
#pragma unroll
    for (int i = 0; i < PPL; ++i) {
      const int pc = p0 + lane + 64 * i;
      xp[i] = pc < p1 ? *reinterpret_cast<const i32x4_t*>(x + (size_t)t * d * 2 + (size_t)pc * 16)
                      : i32x4_t{0, 0, 0, 0};
    }
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < PPL; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) a = fmaf(Piece<MOE_BF16>::get(xp[i], j), Piece<MOE_BF16>::get(wp[i], j), a);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) a += __shfl_xor(a, o);
    if (lane == 0) part[wid][t] = a;
  }
  __syncthreads();
  if (threadIdx.x < T) {
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < kGemvWaves; ++q) s += part[q][threadIdx.x];
    __hip_atomic_store(fp.logits_ws + (size_t)threadIdx.x * E + e, s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();  // part is reused by the next expert
}

template <int PPL>
__device__ __forceinline__ void router_phase(const FusedParams& fp, int bid, int nblk,
                                             float (*part)[kGemvMaxTokens]) {
  for (int e = bid; e < fp.r.E; e += nblk) router_dots<PPL>(fp, e, part);
}

}  // namespace

// TP: token columns a stage holds (T <= TP); D: ring depth.
template <int TP, int D>
__global__ __launch_bounds__(kThreads) void fused_layer_kernel(FusedParams fp) {
  static_assert(D >= 2 && D <= 7, "ring depth: at most 56 loads in flight (vmcnt counts to 63)");
  constexpr int BWIN = TP * 64;  // one piece of the token tile: 4 lane groups x TP columns x 16 bytes
  constexpr int BST = 4 * BWIN;  // the token tile of one stage
  __shared__ __attribute__((aligned(16))) uint8_t ringA[D * kStream * kAWin];
  __shared__ __attribute__((aligned(16))) uint8_t ringB[D * kStream * BST];
  // partial sums: gate/up [2 units in flight][4 waves][4][64]; down [4 waves][2 tiles][4][64]
  __shared__ float red[2 * kStream * 4 * 64];
  __shared__ int s_idx[kMaxSlots];
  __shared__ float s_w[kMaxSlots];
  __shared__ int s_mark[kMaxE];
  __shared__ int s_grp[kMaxE];
  __shared__ int s_meta[4];
  __shared__ float s_part[kWaves][kGemvMaxTokens];

  // stage i of wave w: ringA + (i * kStream + w) * kAWin, ringB + (i * kStream + w) * BST
  const uint32_t la = lds_addr(ringA), lb = lds_addr(ringB);
  const int tid = threadIdx.x, lane = tid & 63, wid = uni(tid >> 6);
  const int bid = blockIdx.x, nblk = gridDim.x;
  const int T = fp.r.T, E = fp.r.E, k = fp.r.k;
  const int d = fp.d, F = fp.F, Fs = fp.Fs, ns = fp.ns;
  const size_t dB = (size_t)d * 2;

  // ---- 0. router GEMM (when the logits are not an input)
  if (fp.w_router) {
    const int ppl = ((d / 8 + kGemvWaves - 1) / kGemvWaves + 63) / 64;
    if (ppl <= 1) router_phase<1>(fp, bid, nblk, s_part);
    else if (ppl <= 2) router_phase<2>(fp, bid, nblk, s_part);
    else if (ppl <= 4) router_phase<4>(fp, bid, nblk, s_part);
    else router_phase<8>(fp, bid, nblk, s_part);
    grid_sync(fp.sync + 0, nblk, fp.err, fp.spin_limit);
  }

  // ---- 1. routing of every token by this workgroup, then the touched
  // experts in index order.  Routing scratch (route_lds_floats(256) floats,
  // 3.5 KB per wave) lives in the weight ring, not in use yet.
  {
    float* kbuf = reinterpret_cast<float*>(ringA + wid * kAWin);
    for (int t = wid; t < T; t += kWaves) {  // uniform per wave
      int my_idx;
      float my_w;
      route_select<kKpl, true>(fp.r, t, kbuf, my_idx, my_w);
      if (lane < k) {
        s_idx[t * k + lane] = my_idx;
        s_w[t * k + lane] = my_w;
      }
    }
  }
  for (int e = tid; e < E; e += kThreads) s_mark[e] = 0;
  __syncthreads();
  for (int i = tid; i < T * k; i += kThreads) s_mark[s_idx[i]] = 1;
  __syncthreads();
  if (wid == 0) {
    int c = 0;
#pragma unroll
    for (int i = 0; i < kKpl; ++i) c += (lane * kKpl + i < E && s_mark[lane * kKpl + i]) ? 1 : 0;
    int inc = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(inc, o);
      if (lane >= o) inc += y;
    }
    int pos = inc - c;
#pragma unroll
    for (int i = 0; i < kKpl; ++i) {
      const int e = lane * kKpl + i;
      if (e < E && s_mark[e]) s_grp[pos++] = e;
    }
    if (lane == 63) s_meta[0] = inc;
  }
  __syncthreads();
  const int Gr = uni(s_meta[0]);    // routed experts with tokens
  const int G = Gr + (ns ? 1 : 0);  // groups: the routed experts, then the shared expert
  const uint8_t* w13 = reinterpret_cast<const uint8_t*>(fp.w13);
  const uint8_t* w2 = reinterpret_cast<const uint8_t*>(fp.w2);
  const uint8_t* ws13 = reinterpret_cast<const uint8_t*>(fp.ws13);
  const uint8_t* ws2 = reinterpret_cast<const uint8_t*>(fp.ws2);
  uint8_t* hr = reinterpret_cast<uint8_t*>(fp.h);  // routed rows [T*k][F]
  uint8_t* hs = hr + (size_t)T * k * F * 2;        // shared rows [T][Fs]
  // slot of token c that chose expert e, or -1
  auto slot_of = [&](int c, int e) {
    int j = -1;
    for (int i = 0; i < k; ++i) j = s_idx[c * k + i] == e ? i : j;
    return j;
  };
  // h row of token c in group g, or -1 when c is not one of its tokens
  auto hrow_of = [&](int c, int g) {
    if (c >= T) return -1;
    if (g >= Gr) return c;
    const int j = slot_of(c, s_grp[g]);
    return j < 0 ? -1 : c * k + j;
  };
  const int r16 = lane & 15, lg = lane >> 4;
  // the token-tile piece this lane loads (lanes < 4 TP): column bc, lane group bg
  const int bc = lane % TP, bg = lane / TP;
  const bool bl = lane < 4 * TP;
  // where this lane's MFMA B operand sits in a token-tile piece
  const int bslot = (lg * TP + (r16 < TP ? r16 : 0)) * 16;

  // ---- 2. gate/up + SwiGLU over this workgroup's units
  const int n8r = F / 8, n8s = ns ? Fs / 8 : 0;
  const long long U = (long long)Gr * n8r + n8s;
  const int ua = (int)(U * bid / nblk), ub = (int)(U * (bid + 1) / nblk);
  const int nunits = ub - ua;
  const int SA = d / 128;  // K-steps of a unit
  // unit u -> group g (Gr: the shared expert), first h column f0
  auto unit_of = [&](int u, int& g, int& f0) {
    if (u < Gr * n8r) {
      g = u / n8r;
      f0 = (u - g * n8r) * 8;
    } else {
      g = Gr;
      f0 = (u - Gr * n8r) * 8;
    }
  };

  if (wid < kStream) {
    const int s0 = wid * SA / kStream, s1 = (wid + 1) * SA / kStream;
    const int cnt = s1 - s0;           // 0 when the model is narrow
    const int nw = cnt > 0 ? cnt : 1;  // such a wave streams one step per unit and drops it
    const int n = nunits * nw;
    const uint8_t* xrow = reinterpret_cast<const uint8_t*>(fp.x) + (size_t)(bc < T ? bc : 0) * dB + 16 * bg;
    int iu = 0, ij = 0, irot = 0, islot = 0;
    const uint8_t* arow = nullptr;
    auto set_unit = [&](int u) {
      int g, f0;
      unit_of(ua + u, g, f0);
      const int Fg = g < Gr ? F : Fs;
      const uint8_t* base = g < Gr ? w13 + (size_t)s_grp[g] * 2 * F * dB : ws13;
      const int row = r16 < 8 ? f0 + r16 : Fg + f0 + r16 - 8;
      arow = base + (size_t)row * dB + 16 * lg;
      // units start their K walk at different steps, so that waves in
      // lockstep spread over the DRAM channels
      irot = cnt > 0 ? (int)(mix((uint32_t)(ua + u)) % (uint32_t)cnt) : 0;
    };
    auto issue = [&]() {
      const int ps = cnt > 0 ? s0 + (ij + irot) % cnt : min(s0, SA - 1);
      const size_t off = (size_t)ps * 256;
      uint8_t* wa = ringA + (islot * kStream + wid) * kAWin;
#pragma unroll
      for (int q = 0; q < 4; ++q) dma16<0>(arow + off + 64 * q, wa + q * 1024);
      if (bl) {
        uint8_t* wb = ringB + (islot * kStream + wid) * BST;
#pragma unroll
        for (int q = 0; q < 4; ++q) dma16<0>(xrow + off + 64 * q, wb + q * BWIN);
      }
      islot = islot + 1 == D ? 0 : islot + 1;
      if (++ij == nw) {
        ij = 0;
        if (++iu < nunits) set_unit(iu);
      }
    };
    if (n > 0) set_unit(0);
    for (int p = 0; p < min(n, D); ++p) issue();
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    int cj = 0, par = 0, cslot = 0;
    for (int p = 0; p < n; ++p) {
      i32x4_t a[4], b[4];
      stage_read(min(D - 1, n - 1 - p), la + (cslot * kStream + wid) * kAWin + lane * 16,
                 lb + (cslot * kStream + wid) * BST + bslot, BWIN, a, b);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a[q]),
                                                      __builtin_bit_cast(bf16x8_t, b[q]), acc, 0, 0, 0);
      cslot = cslot + 1 == D ? 0 : cslot + 1;
      if (++cj == nw) {  // end of this wave's share of a unit
        cj = 0;
        float* dst = red + ((par * kStream + wid) * 4) * 64 + lane;
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[r * 64] = cnt > 0 ? acc[r] : 0.f;
        acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
        par ^= 1;
        lds_barrier();  // the unit's partial sums are in LDS
      }
      if (p + D < n) issue();
    }
  } else {
    // epilogue wave: partial sums -> SwiGLU -> h, one unit per barrier.  Lane
    // l < 32 holds gate rows 4 lg .. 4 lg + 3 of token column r16 (the up
    // rows are the same offsets in lanes l + 32): h columns f0 + 4 lg .. +3.
    for (int u = 0; u < nunits; ++u) {
      lds_barrier();
      if (lane < 32) {
        int g, f0;
        unit_of(ua + u, g, f0);
        const int row = hrow_of(r16, g);
        if (row >= 0) {
          const float* src = red + ((u & 1) * kStream * 4) * 64 + lane;
          uint32_t packed[2];
#pragma unroll
          for (int r = 0; r < 4; r += 2) {
            float hv[2];
#pragma unroll
            for (int e2 = 0; e2 < 2; ++e2) {
              float gs = 0.f, us = 0.f;
#pragma unroll
              for (int w = 0; w < kStream; ++w) {
                gs += src[(w * 4 + r + e2) * 64];
                us += src[(w * 4 + r + e2) * 64 + 32];
              }
              hv[e2] = silu(gs) * us;
            }
            packed[r / 2] = f32_to_bf16_bits(hv[0]) | (f32_to_bf16_bits(hv[1]) << 16);
          }
          uint8_t* dst = g < Gr ? hr + (size_t)row * F * 2 : hs + (size_t)row * Fs * 2;
          const uint64_t v = (uint64_t)packed[0] | ((uint64_t)packed[1] << 32);
          __hip_atomic_store(reinterpret_cast<uint64_t*>(dst + (size_t)(f0 + 4 * lg) * 2), v, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
  }

  // ---- 3. every h of the layer is written
  grid_sync(fp.sync + 1, nblk, fp.err, fp.spin_limit);

  // ---- 4. down + combine over this workgroup's columns [lo, hi) of y
  // (in chunks of at most kMaxTiles 16-row tiles)
  const int Q = d / 4;
  const int wlo = (int)((long long)Q * bid / nblk) * 4, whi = (int)((long long)Q * (bid + 1) / nblk) * 4;
  const int Sr = F / 128, Ss = ns ? Fs / 128 : 0;
  for (int lo = wlo; lo < whi; lo += 16 * kMaxTiles) {  // uniform
    const int hi = min(whi, lo + 16 * kMaxTiles);
    const int nt = (hi - lo + 15) / 16;
    const long long L = (long long)nt * ((long long)Gr * Sr + Ss);
    if (wid < kStream) {
      const long long q0 = L * wid / kStream, q1 = L * (wid + 1) / kStream;
      const int n = (int)(q1 - q0);
      f32x4_t y0 = {0.f, 0.f, 0.f, 0.f}, y1 = {0.f, 0.f, 0.f, 0.f};
      if (n > 0) {
        // position in the sequence (group, 16-row tile, K-step)
        struct Cur {
          int g, tile, s, S;
        };
        auto decode = [&](long long q, Cur& c) {
          const long long rs = (long long)Gr * nt * Sr;
          if (q < rs) {
            c.g = (int)(q / (nt * Sr));
            const int rem = (int)(q - (long long)c.g * nt * Sr);
            c.tile = rem / Sr;
            c.s = rem - c.tile * Sr;
            c.S = Sr;
          } else {
            c.g = Gr;
            const int rem = (int)(q - rs);
            c.tile = rem / Ss;
            c.s = rem - c.tile * Ss;
            c.S = Ss;
          }
        };
        // next step; true when it starts a new (group, tile) segment
        auto advance = [&](Cur& c) {
          if (++c.s < c.S) return false;
          c.s = 0;
          if (++c.tile < nt) return true;
          c.tile = 0;
          ++c.g;
          c.S = c.g < Gr ? Sr : Ss;
          return true;
        };
        Cur ic, cc;
        decode(q0, ic);
        cc = ic;
        const uint8_t* arow = nullptr;
        const uint8_t* hrow = nullptr;
        int hgroup = -1, rot = 0;
        auto set_seg = [&]() {
          const bool sh = ic.g >= Gr;
          const int Fg = sh ? Fs : F;
          const int e = sh ? 0 : s_grp[ic.g];
          int row = lo + 16 * ic.tile + r16;
          row = row < hi ? row : lo;  // rows past the slice: a valid duplicate, never stored
          arow = (sh ? ws2 : w2 + (size_t)e * d * F * 2) + (size_t)row * Fg * 2 + 16 * lg;
          if (ic.g != hgroup) {
            hgroup = ic.g;
            const int r = hrow_of(bc, ic.g);  // unused columns read row 0
            hrow = (r < 0 ? hr : sh ? hs + (size_t)r * Fs * 2 : hr + (size_t)r * F * 2) + 16 * bg;
          }
          rot = (int)(mix((uint32_t)((sh ? kMaxE : e) * 4096 + lo / 16 + ic.tile)) % (uint32_t)ic.S);
        };
        set_seg();
        int islot = 0, cslot = 0;
        auto issue = [&]() {
          const int ps = ic.s + rot < ic.S ? ic.s + rot : ic.s + rot - ic.S;
          const size_t off = (size_t)ps * 256;
          uint8_t* wa = ringA + (islot * kStream + wid) * kAWin;
#pragma unroll
          for (int q = 0; q < 4; ++q) dma16<0>(arow + off + 64 * q, wa + q * 1024);
          if (bl) {
            uint8_t* wb = ringB + (islot * kStream + wid) * BST;
#pragma unroll
            for (int q = 0; q < 4; ++q) dma16<kSc1>(hrow + off + 64 * q, wb + q * BWIN);
          }
          islot = islot + 1 == D ? 0 : islot + 1;
          if (advance(ic) && ic.g < G) set_seg();
        };
        for (int p = 0; p < min(n, D); ++p) issue();
        // this lane's token column in the consume cursor's group: taken, gate weight
        bool fon = false;
        float fw = 0.f;
        auto set_fold = [&]() {
          const int r = hrow_of(r16, cc.g);
          fon = r >= 0;
          fw = !fon ? 0.f : cc.g < Gr ? s_w[r] : 1.f;
        };
        set_fold();
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        for (int p = 0; p < n; ++p) {
          i32x4_t a[4], b[4];
          stage_read(min(D - 1, n - 1 - p), la + (cslot * kStream + wid) * kAWin + lane * 16,
                     lb + (cslot * kStream + wid) * BST + bslot, BWIN, a, b);
#pragma unroll
          for (int q = 0; q < 4; ++q)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a[q]),
                                                          __builtin_bit_cast(bf16x8_t, b[q]), acc, 0, 0, 0);
          cslot = cslot + 1 == D ? 0 : cslot + 1;
          if (cc.s == cc.S - 1 || p + 1 == n) {
            // end of a segment (or of this wave's share of one): the expert's
            // output for these columns of y, times the token's gate weight
            if (fon) {
              if (cc.tile == 0) {
#pragma unroll
                for (int r = 0; r < 4; ++r) y0[r] = fmaf(fw, acc[r], y0[r]);
              } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) y1[r] = fmaf(fw, acc[r], y1[r]);
              }
            }
            acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
          }
          if (p + 1 < n) {
            const int g0 = cc.g;
            advance(cc);
            if (cc.g != g0) set_fold();
          }
          if (p + D < n) issue();
        }
      }
      float* dst = red + (wid * kMaxTiles * 4) * 64 + lane;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        dst[r * 64] = y0[r];
        dst[(4 + r) * 64] = y1[r];
      }
    }
    lds_barrier();
    if (wid == kEpi) {
      // lane: rows 4 lg .. 4 lg + 3 of each tile, token column r16
      for (int t = 0; t < nt; ++t) {
        const int row = lo + 16 * t + 4 * lg;
        if (r16 < T && row < hi) {
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float s = 0.f;
#pragma unroll
            for (int w = 0; w < kStream; ++w) s += red[((w * kMaxTiles + t) * 4 + r) * 64 + lane];
            v[r] = s;
          }
          const uint32_t lo2 = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16);
          const uint32_t hi2 = f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16);
          *reinterpret_cast<uint2*>(fp.y + (size_t)r16 * d + row) = make_uint2(lo2, hi2);
        }
      }
    }
    lds_barrier();  // red is rewritten by the next chunk
  }
  if (wid == kEpi) {
    // ---- exit: the last workgroup out zeroes the counters for the next call
    if (lane == 0) {
      const int done = __hip_atomic_fetch_add(fp.sync + 3, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (done == nblk - 1)
        for (int i = 0; i < 4; ++i) __hip_atomic_store(fp.sync + i, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

namespace {

template <int TP, int D>
hipError_t launch_fused_shape(const FusedParams& p, int nblk, hipStream_t stream) {
  hipLaunchKernelGGL((fused_layer_kernel<TP, D>), dim3(nblk), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

// Every workgroup must be resident at once (grid barriers): one per CU, and
// the launch is refused unless the occupancy calculation allows one per CU
// for every instantiation (constant per device model, computed once).
Residency fused_residency() {
  static const Residency occ = [] {
    Residency o{};
    int dev = 0, c = 0;
    if (hipGetDevice(&dev) != hipSuccess) return o;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return o;
    int n = 1 << 30;
    const void* kernels[] = {(const void*)fused_layer_kernel<1, 7>, (const void*)fused_layer_kernel<4, 6>,
                             (const void*)fused_layer_kernel<8, 5>, (const void*)fused_layer_kernel<16, 4>};
    for (const void* kfn : kernels) {
      int m = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&m, kfn, kThreads, 0) != hipSuccess) return o;
      n = m < n ? m : n;
    }
    o.per_cu = n;
    o.cus = c;
    o.ok = n >= 1 && c >= 1;
    return o;
  }();
  return occ;
}

}  // namespace

int fused_grid() {
  const Residency occ = fused_residency();
  return occ.ok ? occ.cus : 0;
}

bool fused_shape_ok(int T, int k, int E, int d, int F, int Fs) {
  if (T < 1 || T > kMaxT || k < 1 || k > 64 || T * k > kMaxSlots || E < 1 || E > kMaxE) return false;
  return d >= 128 && d % 128 == 0 && F >= 128 && F % 128 == 0 && Fs >= 0 && Fs % 128 == 0;
}

hipError_t launch_fused(const FusedParams& p, hipStream_t stream) {
  const int nblk = fused_grid();
  if (nblk < 1) return hipErrorInvalidDevice;
  if (!fused_shape_ok(p.r.T, p.r.k, p.r.E, p.d, p.F, p.ns ? p.Fs : 0)) return hipErrorInvalidValue;
  const int T = p.r.T;
  if (T <= 1) return launch_fused_shape<1, 7>(p, nblk, stream);
  if (T <= 4) return launch_fused_shape<4, 6>(p, nblk, stream);
  if (T <= 8) return launch_fused_shape<8, 5>(p, nblk, stream);
  return launch_fused_shape<16, 4>(p, nblk, stream);
}

}  // namespace moe
