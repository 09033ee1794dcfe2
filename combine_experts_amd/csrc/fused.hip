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
//     experts and of the shared expert are split over the grid in contiguous
//     runs of equal cost (weight rows plus the group's token columns); the
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
//     A workgroup that owns at most 8 columns packs two K-steps into each
//     16-row weight tile, so that no tile row is a duplicate.
//
// Streaming: each streaming wave runs a ring of DA (gate/up) or DB (down)
// stages in LDS.  A stage is one 256-byte K-step of a 16-row weight tile (4
// KB) and of the token tile (16 bytes per lane group and token column; only
// the columns of the group's own tokens are loaded), brought in by
// direct-to-LDS loads (global_load_lds_dwordx4), so the stages in flight need
// no staging registers.  Before a stage is read the wave waits (s_waitcnt)
// until only the loads issued after the stage's own are outstanding; the
// streaming waves issue no other vector-memory operation inside their loops
// (no stores, no scratch), so the count is exact.  Both passes stream at
// about 20 GB/s per CU (5 TB/s over the chip).
//
// Handoff between workgroups: h (and the router's logits) are written with
// device-scope stores and read with device-scope loads, so a grid barrier
// needs no cache write-back or invalidate (measured: an agent-scope release
// and acquire per workgroup cost 12-16 us per barrier): each wave that stored
// waits until its stores are done, then the epilogue wave counts the
// workgroup in (two-level counters) and waits for the release flag.  The
// wait is bounded by spin_limit; when it gives up it sets the error word and
// lets the workgroup go on, so every wave always reaches the end of the
// kernel.  The workgroup that counts out last zeroes the counters and flags
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

// One ring stage -> MFMA operands: wait until at most 4 n4 of this wave's
// vector-memory operations are in flight (the loads issued after the
// stage's own), read the stage's four weight pieces (wa, 1 KB apart) and its
// 4 P token pieces (wb0 + j bwin), and wait for the reads.  One asm block, so
// the compiler neither adds a wait of its own (it cannot tell which ring slot
// a direct-to-LDS load writes) nor uses the outputs before the reads are done.
#define MOE_READ1(M)                                                                              \
  asm volatile("s_waitcnt vmcnt(" #M ")\n\t"                                                      \
               "ds_read_b128 %0, %8\n\tds_read_b128 %1, %8 offset:1024\n\t"                        \
               "ds_read_b128 %2, %8 offset:2048\n\tds_read_b128 %3, %8 offset:3072\n\t"            \
               "ds_read_b128 %4, %9\n\tds_read_b128 %5, %10\n\t"                                   \
               "ds_read_b128 %6, %11\n\tds_read_b128 %7, %12\n\t"                                  \
               "s_waitcnt lgkmcnt(0)"                                                              \
               : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3]), "=&v"(b[0]), "=&v"(b[1]),       \
                 "=&v"(b[2]), "=&v"(b[3])                                                          \
               : "v"(wa), "v"(wb0), "v"(wb0 + bwin), "v"(wb0 + 2 * bwin), "v"(wb0 + 3 * bwin)      \
               : "memory")
#define MOE_READ2(M)                                                                              \
  asm volatile("s_waitcnt vmcnt(" #M ")\n\t"                                                      \
               "ds_read_b128 %0, %12\n\tds_read_b128 %1, %12 offset:1024\n\t"                      \
               "ds_read_b128 %2, %12 offset:2048\n\tds_read_b128 %3, %12 offset:3072\n\t"          \
               "ds_read_b128 %4, %13\n\tds_read_b128 %5, %14\n\t"                                  \
               "ds_read_b128 %6, %15\n\tds_read_b128 %7, %16\n\t"                                  \
               "ds_read_b128 %8, %17\n\tds_read_b128 %9, %18\n\t"                                  \
               "ds_read_b128 %10, %19\n\tds_read_b128 %11, %20\n\t"                                \
               "s_waitcnt lgkmcnt(0)"                                                              \
               : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3]), "=&v"(b[0]), "=&v"(b[1]),       \
                 "=&v"(b[2]), "=&v"(b[3]), "=&v"(b[4]), "=&v"(b[5]), "=&v"(b[6]), "=&v"(b[7])        \
               : "v"(wa), "v"(wb0), "v"(wb0 + bwin), "v"(wb0 + 2 * bwin), "v"(wb0 + 3 * bwin),     \
                 "v"(wb0 + 4 * bwin), "v"(wb0 + 5 * bwin), "v"(wb0 + 6 * bwin), "v"(wb0 + 7 * bwin) \
               : "memory")
#define MOE_READ_CASES(R)                                                                         \
  switch (n4) {                                                                                   \
    case 0: R(0); break;   case 1: R(4); break;   case 2: R(8); break;   case 3: R(12); break;     \
    case 4: R(16); break;  case 5: R(20); break;  case 6: R(24); break;  case 7: R(28); break;     \
    case 8: R(32); break;  case 9: R(36); break;  case 10: R(40); break; case 11: R(44); break;    \
    case 12: R(48); break; case 13: R(52); break; case 14: R(56); break; default: R(60); break;    \
  }

template <int P>
__device__ __forceinline__ void stage_read(int n4, uint32_t wa, uint32_t wb0, uint32_t bwin, i32x4_t (&a)[4],
                                           i32x4_t (&b)[4 * P]) {
  if constexpr (P == 1) {
    MOE_READ_CASES(MOE_READ1)
  } else {
    MOE_READ_CASES(MOE_READ2)
  }
}
#undef MOE_READ_CASES
#undef MOE_READ2
#undef MOE_READ1

// LDS address of a shared-memory pointer
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Workgroup barrier that orders LDS only (a fence would wait for every load
// in flight); the memory clobber keeps the compiler from moving accesses
// across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Grid-wide barrier of the resident workgroups, two levels deep.  The waves
// that stored data for other workgroups (all of them, or with all_store
// false only the epilogue wave)
// first wait until their own (device-scope) stores are done; then the
// epilogue wave's first lane counts the workgroup in on its group's counter
// (workgroup b is in group b % 8, the counters 256 bytes apart), the last
// arrival of a group counts the group in at the top, the last group raises
// the release flag, and every workgroup waits for the flag to read exactly 1
// (a word no arrival writes to, so the waiting does not slow the arrivals;
// counters or a flag left non-zero by an interrupted call make the wait run
// out, setting the error word, rather than pass early).  Measured on 256
// workgroups arriving together: 1.7 us per barrier, against 4.3 us when
// every workgroup polls per-workgroup flags and 3.8 us for a single counter.
// Block layout (ints): [0] top count, [64] release flag, [128 + 64 g] group
// g's count.
constexpr int kBarGroups = 8;
static_assert(128 + 64 * kBarGroups <= kFusedBarWords, "barrier block");

__device__ __forceinline__ void grid_sync(int* bar, int nblk, int* err, int spin_limit, bool all_store) {
  if (all_store || (threadIdx.x >> 6) == kEpi) wait_vm<0>();
  lds_barrier();
  if (threadIdx.x == 64 * kEpi) {
    const int g = blockIdx.x % kBarGroups;
    const int gsize = (nblk - g + kBarGroups - 1) / kBarGroups;  // workgroups b < nblk with b % 8 == g
    const int groups = nblk < kBarGroups ? nblk : kBarGroups;
    if (__hip_atomic_fetch_add(bar + 128 + 64 * g, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gsize - 1 &&
        __hip_atomic_fetch_add(bar, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == groups - 1)
      __hip_atomic_store(bar + 64, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int n = 0; __hip_atomic_load(bar + 64, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 1; ++n) {
      if (n >= spin_limit) {
        __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  lds_barrier();
}

__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Relative cost of one gate/up unit whose group has n token columns: 16 weight
// rows plus n token columns at 3/4 of a row each, in quarters of a row.
__device__ __forceinline__ int unit_cost(int n) { return 64 + 3 * n; }

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

// TP: token columns a stage holds (T <= TP); DA, DB: ring depth of the
// gate/up and the down pass; P: K-steps per weight tile in the down pass (2
// when a workgroup owns at most 8 columns of y: the tile's rows 8-15 hold the
// same columns one K-step further, so no tile row is wasted).
template <int TP, int DA, int DB, int P>
__global__ __launch_bounds__(kThreads) void fused_layer_kernel(FusedParams fp) {
  // at most 63 vector-memory operations in flight per wave (vmcnt counts to 63)
  static_assert(DA >= 2 && (4 + (16 * TP + 63) / 64) * DA <= 63 && DB >= 2 && DB <= DA &&
                    (4 + (16 * P * TP + 63) / 64) * DB <= 63, "ring depth");
  static_assert(P == 1 || P == 2, "pack");
  constexpr int NBA = (16 * TP + 63) / 64;      // token-tile loads per gate/up stage
  constexpr int NBB = (16 * P * TP + 63) / 64;  // token-tile loads per down stage
  constexpr int NSA = 4 + NBA, NSB = 4 + NBB;   // all loads of a stage
  constexpr int BWIN = TP * 64;   // one piece of the token tile: 4 lane groups x TP columns x 16 bytes
  constexpr int BST = 4 * BWIN;   // the token tile of one K-step
  constexpr int BSTP = P * BST;   // the token tiles of one down-pass stage
  constexpr int RB = (DA * BST > DB * BSTP ? DA * BST : DB * BSTP) * kStream;
  __shared__ __attribute__((aligned(16))) uint8_t ringA[DA * kStream * kAWin];
  __shared__ __attribute__((aligned(16))) uint8_t ringB[RB];
  // partial sums: gate/up [2 units in flight][4 waves][64 lanes][4]; down [4 waves][2 tiles][64][4]
  __shared__ __attribute__((aligned(16))) float red[2 * kStream * 4 * 64];
  __shared__ int s_idx[kMaxSlots];
  __shared__ float s_w[kMaxSlots];
  __shared__ int s_mark[kMaxE];
  __shared__ int s_grp[kMaxE];
  __shared__ int s_gcost[kMaxE + 1];  // cost of group g's gate/up units
  __shared__ int s_gpre[kMaxE + 1];   // cost of the groups before g
  __shared__ int s_meta[4];
  __shared__ float s_part[kWaves][kGemvMaxTokens];

  // stage slot i of wave w: ringA + (i * kStream + w) * kAWin, ringB + (i * kStream + w) * BST (gate/up)
  // or BSTP (down); stage j of a wave's sequence is in slot j % depth
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
    grid_sync(fp.bar0, nblk, fp.err, fp.spin_limit, true);
  }

  for (int e = tid; e < E; e += kThreads) s_mark[e] = 0;  // read after the barrier that follows routing

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
  __syncthreads();
  const int n8r = F / 8, n8s = ns ? Fs / 8 : 0;  // gate/up units (8 columns of h) per group
  if (wid == 0) {
    // one wave: count each expert's tokens (a token picks an expert at most
    // once), list the experts with tokens in index order, and the prefix of
    // the groups' gate/up cost (see below)
    for (int i = lane; i < T * k; i += 64) atomicAdd(&s_mark[s_idx[i]], 1);
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
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
    const int gr = __shfl(inc, 63);
#pragma unroll
    for (int i = 0; i < kKpl; ++i) {
      const int e = lane * kKpl + i;
      if (e < E && s_mark[e]) {
        s_grp[pos] = e;
        s_gcost[pos] = n8r * unit_cost(s_mark[e]);
        ++pos;
      }
    }
    if (lane == 0 && ns) s_gcost[gr] = n8s * unit_cost(T);
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    // exclusive prefix of the group costs over the gr + ns groups (<= 257)
    const int ng = gr + (ns ? 1 : 0);
    int v[5], sum = 0;
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      const int g = lane * 5 + i;
      v[i] = g < ng ? s_gcost[g] : 0;
      sum += v[i];
    }
    int inc2 = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(inc2, o);
      if (lane >= o) inc2 += y;
    }
    int run = inc2 - sum;
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      const int g = lane * 5 + i;
      if (g < ng) s_gpre[g] = run;
      run += v[i];
    }
    if (lane == 63) {
      s_meta[0] = gr;
      s_meta[1] = inc2;  // total cost
    }
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
  // Token tiles in LDS: 16-byte slot ((j 4 + q) 4 + g) TP + c holds K-step j
  // of the stage, piece q (bytes 64 q + 16 g of the 256-byte step) of token
  // column c; the MFMA B operand of lane (lg, r16) for piece q of step j is
  // slot ((j 4 + q) 4 + lg) TP + r16.  The loads fill the slots densely, 64
  // per instruction (slot 64 i + lane), so a stage of TP columns and NB steps
  // takes 16 TP NB / 64 load instructions rather than 4 per step.  Only the
  // columns of the group's own tokens are loaded; every instruction covers all
  // TP columns and every group has a token, so each instruction still issues
  // (the wait counts above count instructions).  The other columns keep stale
  // LDS: their products are never used.
  const int bc = lane % TP;  // token column of every slot this lane loads
  auto tile_off = [&](int i) {
    const int sl = 64 * i + lane, j = sl / (16 * TP), q = (sl / (4 * TP)) % 4, g = (sl / TP) % 4;
    return j * 256 + 64 * q + 16 * g;
  };
  int boA[NBA], boB[NBB];
#pragma unroll
  for (int i = 0; i < NBA; ++i) boA[i] = tile_off(i);
#pragma unroll
  for (int i = 0; i < NBB; ++i) boB[i] = tile_off(i);
  // where this lane's MFMA B operand sits in a step's token tile
  const int bslot = (lg * TP + (r16 < TP ? r16 : 0)) * 16;

  // ---- 2. gate/up + SwiGLU over this workgroup's units.  A unit of a group
  // with n tokens streams 16 weight rows and n token columns per K-step; the
  // units are split over the grid in contiguous runs of equal total cost
  // unit_cost(n) (measured: a token column costs about 3/4 of a weight row
  // per step), so that groups with many tokens (the shared expert) do not
  // leave their workgroups behind.  Workgroup b takes the units whose start
  // (the cost of the units before them) lies in [b C / nblk, (b+1) C / nblk).
  const long long U = (long long)Gr * n8r + n8s;
  const long long Ctot = uni(s_meta[1]);
  auto first_unit = [&](long long X) -> int {  // first unit starting at or after cost X
    if (X >= Ctot) return (int)U;
    int ng = 0;  // groups starting at or before X
    for (int i = 0; i < 5; ++i) {
      const int g = lane * 5 + i;
      ng += __popcll(__ballot(g < G && s_gpre[g] <= X));
    }
    const int g = ng - 1;
    const int cg = unit_cost(g < Gr ? uni(s_mark[uni(s_grp[g])]) : T);
    const long long before = (X - uni(s_gpre[g]) + cg - 1) / cg;  // units of g that start before X
    return (int)((long long)g * n8r + before);
  };
  const int ua = first_unit(Ctot * bid / nblk), ub = first_unit(Ctot * (bid + 1) / nblk);
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
    const uint8_t* xrow = reinterpret_cast<const uint8_t*>(fp.x) + (size_t)(bc < T ? bc : 0) * dB;
    int iu = 0, ij = 0, irot = 0, islot = 0;
    const uint8_t* arow = nullptr;
    bool bon = false;  // this lane's token column is one of the unit's tokens (others are not loaded)
    auto set_unit = [&](int u) {
      int g, f0;
      unit_of(ua + u, g, f0);
      bon = hrow_of(bc, g) >= 0;
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
      uint8_t* wb = ringB + (islot * kStream + wid) * BST;
#pragma unroll
      for (int i = 0; i < NBA; ++i)
        if (64 * i + lane < 16 * TP && bon) dma16<0>(xrow + off + boA[i], wb + 1024 * i);
      islot = islot + 1 == DA ? 0 : islot + 1;
      if (++ij == nw) {
        ij = 0;
        if (++iu < nunits) set_unit(iu);
      }
    };
    if (n > 0) set_unit(0);
    for (int p = 0; p < min(n, DA); ++p) issue();
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    int cj = 0, par = 0, cslot = 0;
    for (int p = 0; p < n; ++p) {
      i32x4_t a[4], b[4];
      stage_read<1>(NSA * min(DA - 1, n - 1 - p) / 4, la + (cslot * kStream + wid) * kAWin + lane * 16,
                    lb + (cslot * kStream + wid) * BST + bslot, BWIN, a, b);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a[q]),
                                                      __builtin_bit_cast(bf16x8_t, b[q]), acc, 0, 0, 0);
      cslot = cslot + 1 == DA ? 0 : cslot + 1;
      if (++cj == nw) {  // end of this wave's share of a unit
        cj = 0;
        *reinterpret_cast<f32x4_t*>(red + ((par * kStream + wid) * 64 + lane) * 4) =
            cnt > 0 ? acc : f32x4_t{0.f, 0.f, 0.f, 0.f};
        acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
        par ^= 1;
        lds_barrier();  // the unit's partial sums are in LDS
      }
      if (p + DA < n) issue();
    }
  } else {
    // epilogue wave: partial sums -> SwiGLU -> h, one unit per barrier.  Lane
    // l < 32 holds gate rows 4 lg .. 4 lg + 3 of token column r16 (the up
    // rows are the same offsets in lanes l + 32): h columns f0 + 4 lg .. +3.
    // The unit's h row is looked up before its barrier, off the critical path.
    for (int u = 0; u < nunits; ++u) {
      int g, f0, row = -1;
      if (lane < 32) {
        unit_of(ua + u, g, f0);
        row = hrow_of(r16, g);
      }
      lds_barrier();
      if (row >= 0) {
        const float* src = red + ((u & 1) * kStream * 64 + lane) * 4;
        f32x4_t gs = {0.f, 0.f, 0.f, 0.f}, us = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < kStream; ++w) {
          const f32x4_t gw = *reinterpret_cast<const f32x4_t*>(src + w * 256);
          const f32x4_t uw = *reinterpret_cast<const f32x4_t*>(src + w * 256 + 128);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            gs[r] += gw[r];
            us[r] += uw[r];
          }
        }
        uint32_t packed[2];
#pragma unroll
        for (int r = 0; r < 4; r += 2)
          packed[r / 2] = f32_to_bf16_bits(silu(gs[r]) * us[r]) | (f32_to_bf16_bits(silu(gs[r + 1]) * us[r + 1]) << 16);
        uint8_t* dst = g < Gr ? hr + (size_t)row * F * 2 : hs + (size_t)row * Fs * 2;
        const uint64_t v = (uint64_t)packed[0] | ((uint64_t)packed[1] << 32);
        __hip_atomic_store(reinterpret_cast<uint64_t*>(dst + (size_t)(f0 + 4 * lg) * 2), v, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }

  // ---- 3. every h of the layer is written; 4. down + combine over this
  // workgroup's columns [wlo, whi) of y, in chunks of at most CHR columns.
  // (Issuing the first weight tiles of the down pass before the barrier was
  // measured no faster: the burst of loads delays the barrier's atomics by
  // about as much as it saves in the down pass.)
  constexpr int RT = 16 / P;            // y columns per tile
  constexpr int CHR = P == 1 ? 16 * kMaxTiles : RT;
  const int Q = d / 4;
  const int wlo = (int)((long long)Q * bid / nblk) * 4, whi = (int)((long long)Q * (bid + 1) / nblk) * 4;
  const int Sr = F / 128 / P, Ss = ns ? Fs / 128 / P : 0;  // stages per (group, tile) segment
  // position in the sequence (group, tile, stage)
  struct Cur {
    int g, tile, s, S;
  };
  int lo = wlo, hi = min(whi, wlo + CHR), nt = 0, n = 0;
  Cur ic{}, cc{};
  const uint8_t* arow = nullptr;
  const uint8_t* hrow = nullptr;
  int hgroup = -1, rot = 0, islot = 0, cslot = 0;
  auto advance = [&](Cur& c) {  // next stage; true when it starts a new segment
    if (++c.s < c.S) return false;
    c.s = 0;
    if (++c.tile < nt) return true;
    c.tile = 0;
    ++c.g;
    c.S = c.g < Gr ? Sr : Ss;
    return true;
  };
  auto set_seg = [&]() {
    const bool sh = ic.g >= Gr;
    const int Fg = sh ? Fs : F;
    const int e = sh ? 0 : s_grp[ic.g];
    int row = lo + RT * ic.tile + (P == 2 ? (r16 & 7) : r16);
    row = row < hi ? row : lo;  // columns past the chunk: a valid duplicate, never stored
    // packed tiles: rows 8-15 hold the same columns one K-step further
    arow = (sh ? ws2 : w2 + (size_t)e * d * F * 2) + (size_t)row * Fg * 2 + 16 * lg + (P == 2 && r16 >= 8 ? 256 : 0);
    if (ic.g != hgroup) {
      hgroup = ic.g;
      const int r = hrow_of(bc, ic.g);  // columns of none of the group's tokens are not loaded
      hrow = r < 0 ? nullptr : sh ? hs + (size_t)r * Fs * 2 : hr + (size_t)r * F * 2;
    }
    rot = (int)(mix((uint32_t)((sh ? kMaxE : e) * 4096 + lo / 16 + ic.tile)) % (uint32_t)ic.S);
  };
  // this wave's share of the chunk [lo, hi): n stages from cursor position q0
  auto setup_chunk = [&]() {
    nt = (hi - lo + RT - 1) / RT;
    const long long L = (long long)nt * ((long long)Gr * Sr + Ss);
    const long long q0 = L * wid / kStream, q1 = L * (wid + 1) / kStream;
    n = (int)(q1 - q0);
    if (n <= 0) return;
    const long long rs = (long long)Gr * nt * Sr;
    if (q0 < rs) {
      ic.g = (int)(q0 / (nt * Sr));
      const int rem = (int)(q0 - (long long)ic.g * nt * Sr);
      ic.tile = rem / Sr;
      ic.s = rem - ic.tile * Sr;
      ic.S = Sr;
    } else {
      ic.g = Gr;
      const int rem = (int)(q0 - rs);
      ic.tile = rem / Ss;
      ic.s = rem - ic.tile * Ss;
      ic.S = Ss;
    }
    cc = ic;
    hgroup = -1;
    set_seg();
    islot = cslot = 0;
  };
  // the issue cursor's stage: weight source (per lane) and token source (per
  // loading lane); then the cursor moves on
  auto stage_src = [&](const uint8_t*& asrc, const uint8_t*& bsrc) {
    const int ps = ic.s + rot < ic.S ? ic.s + rot : ic.s + rot - ic.S;
    asrc = arow + (size_t)(P * ps) * 256;
    bsrc = hrow ? hrow + (size_t)(P * ps) * 256 : nullptr;
    if (advance(ic) && ic.g < G) set_seg();
  };
  auto dmaA = [&](int slot, const uint8_t* asrc) {
    uint8_t* wa = ringA + (slot * kStream + wid) * kAWin;
#pragma unroll
    for (int q = 0; q < 4; ++q) dma16<0>(asrc + 64 * q, wa + q * 1024);
  };
  auto dmaB = [&](int slot, const uint8_t* bsrc) {
    uint8_t* wb = ringB + (slot * kStream + wid) * BSTP;
#pragma unroll
    for (int i = 0; i < NBB; ++i)
      if (64 * i + lane < 16 * P * TP && bsrc) dma16<kSc1>(bsrc + boB[i], wb + 1024 * i);
  };
  constexpr int NS = NSB;  // loads of a stage

  grid_sync(fp.bar1, nblk, fp.err, fp.spin_limit, false);
  // count this workgroup out of the barriers now; the answer is needed only
  // at the end, so its round trip overlaps the down pass
  int exit_rank = 0;
  if (tid == 64 * kEpi) exit_rank = __hip_atomic_fetch_add(fp.sync + 3, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  for (; lo < whi; lo += CHR, hi = min(whi, lo + CHR)) {  // uniform
    nt = (hi - lo + RT - 1) / RT;
    if (wid < kStream) {
      f32x4_t y0 = {0.f, 0.f, 0.f, 0.f}, y1 = {0.f, 0.f, 0.f, 0.f};
      setup_chunk();
      for (int i = 0; i < min(n, DB); ++i) {  // stage i in slot i
        const uint8_t* asrc;
        const uint8_t* bsrc;
        stage_src(asrc, bsrc);
        dmaA(i, asrc);
        dmaB(i, bsrc);
      }
      if (n > 0) {
        // this lane's token column in the consume cursor's group: taken, gate weight
        bool fon = false;
        float fw = 0.f;
        auto set_fold = [&]() {
          const int r = hrow_of(r16, cc.g);
          fon = r >= 0;
          fw = !fon ? 0.f : cc.g < Gr ? s_w[r] : 1.f;
        };
        set_fold();
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f}, acc2 = {0.f, 0.f, 0.f, 0.f};
        for (int p = 0; p < n; ++p) {
          const int m = NS * min(DB - 1, n - 1 - p);  // loads issued after this stage's last one
          i32x4_t a[4], b[4 * P];
          stage_read<P>(m / 4, la + (cslot * kStream + wid) * kAWin + lane * 16,
                        lb + (cslot * kStream + wid) * BSTP + bslot, BWIN, a, b);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a[q]),
                                                          __builtin_bit_cast(bf16x8_t, b[q]), acc, 0, 0, 0);
            if constexpr (P == 2)
              acc2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a[q]),
                                                             __builtin_bit_cast(bf16x8_t, b[4 + q]), acc2, 0, 0, 0);
          }
          cslot = cslot + 1 == DB ? 0 : cslot + 1;
          if (cc.s == cc.S - 1 || p + 1 == n) {
            // end of a segment (or of this wave's share of one): the expert's
            // output for these columns of y, times the token's gate weight
            if constexpr (P == 2) {
              // rows 0-7 (lanes 0-31) of acc and rows 8-15 (lanes 32-63) of
              // acc2 are the same columns at even and odd K-steps
#pragma unroll
              for (int r = 0; r < 4; ++r) acc[r] += __shfl_down(acc2[r], 32);
              acc2 = f32x4_t{0.f, 0.f, 0.f, 0.f};
            }
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
          if (p + DB < n) {
            const uint8_t* asrc;
            const uint8_t* bsrc;
            const int slot = islot;
            islot = islot + 1 == DB ? 0 : islot + 1;
            stage_src(asrc, bsrc);
            dmaA(slot, asrc);
            dmaB(slot, bsrc);
          }
        }
      }
      *reinterpret_cast<f32x4_t*>(red + ((wid * kMaxTiles + 0) * 64 + lane) * 4) = y0;
      *reinterpret_cast<f32x4_t*>(red + ((wid * kMaxTiles + 1) * 64 + lane) * 4) = y1;
    }
    lds_barrier();
    if (wid == kEpi) {
      // lane: columns 4 lg .. 4 lg + 3 of each tile, token r16
      for (int t = 0; t < nt; ++t) {
        const int row = lo + RT * t + 4 * lg;
        if (r16 < T && row < hi && 4 * lg < RT) {
          f32x4_t v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int w = 0; w < kStream; ++w) {
            const f32x4_t pw = *reinterpret_cast<const f32x4_t*>(red + ((w * kMaxTiles + t) * 64 + lane) * 4);
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] += pw[r];
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
    // ---- exit: the workgroup that counted in last after the final barrier
    // zeroes the flags of both barriers and the count for the next call
    // (every workgroup had finished waiting on them before counting in)
    if (__shfl(exit_rank, 0) == nblk - 1 && lane < 2 + kBarGroups) {
      // top count, flag, group counts of both barriers; the exit count
      __hip_atomic_store(fp.bar0 + 64 * lane, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(fp.bar1 + 64 * lane, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (lane == 0) __hip_atomic_store(fp.sync + 3, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

namespace {

template <int TP, int DA, int DB, int P>
hipError_t launch_fused_shape(const FusedParams& p, int nblk, hipStream_t stream) {
  hipLaunchKernelGGL((fused_layer_kernel<TP, DA, DB, P>), dim3(nblk), dim3(kThreads), 0, stream, p);
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
    const void* kernels[] = {
        (const void*)fused_layer_kernel<1, 8, 8, 1>, (const void*)fused_layer_kernel<1, 8, 8, 2>,
        (const void*)fused_layer_kernel<4, 7, 7, 1>, (const void*)fused_layer_kernel<4, 6, 6, 2>,
        (const void*)fused_layer_kernel<8, 6, 6, 1>, (const void*)fused_layer_kernel<8, 5, 4, 2>,
        (const void*)fused_layer_kernel<16, 4, 4, 1>};
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
  // two K-steps per down-pass tile when a workgroup owns at most 8 columns
  // of y and every expert's K-steps pair up
  const int Q = p.d / 4, per = (Q + nblk - 1) / nblk;
  const bool pack = 4 * per <= 8 && (p.F / 128) % 2 == 0 && (!p.ns || (p.Fs / 128) % 2 == 0);
  const int T = p.r.T;
  if (T <= 1) return pack ? launch_fused_shape<1, 8, 8, 2>(p, nblk, stream) : launch_fused_shape<1, 8, 8, 1>(p, nblk, stream);
  if (T <= 4) return pack ? launch_fused_shape<4, 6, 6, 2>(p, nblk, stream) : launch_fused_shape<4, 7, 7, 1>(p, nblk, stream);
  if (T <= 8) return pack ? launch_fused_shape<8, 5, 4, 2>(p, nblk, stream) : launch_fused_shape<8, 6, 6, 1>(p, nblk, stream);
  return launch_fused_shape<16, 4, 4, 1>(p, nblk, stream);
}

}  // namespace moe
