// Grouped expert GEMMs for prefill-sized batches (bf16).  "7.13 Serving
// Mixture-of-Experts", section "Prefill vs. Decode": with many tokens per
// expert the grouped GEMM is fat and each weight tile can be reused across
// many token rows.
//
// Design (gfx950): work item = (group, 128-row token tile, feature tile).
// A workgroup of WR/32 waves computes a WR x 128 block: WR weight rows (the
// gate and up rows of WR/2 features in the gated pass, WR output features in
// the plain pass) against 128 token rows, K in steps of 64.  Each step's tiles
// go straight from HBM into LDS with direct-to-LDS loads
// (global_load_lds_dwordx4: each lane's 16 bytes land at lane x 16 of a
// 1 KB wave window), three steps deep, with no staging registers and no LDS
// store instructions.  A lane picks which 16-byte chunk of its row it fetches
// so that the rows land XOR-swizzled and the MFMA operand reads are free of
// bank conflicts.  The three stages are separate LDS arrays: the compiler can
// then tell a read of one stage from the loads still landing in the others
// and does not drain them; the per-step barrier waits (by count) only for the
// wave's own loads of the stage about to be read.  Each wave owns a 64 x 64
// block (4 x 4 MFMA tiles) and, in the gated pass, holds matching gate and up
// columns, so SwiGLU is applied in registers (MFMA:
// v_mfma_f32_16x16x32_bf16).  WR = 256 when the feature count allows: one
// token tile then feeds twice as many weight rows.  Items are ordered (group,
// feature tile, token tile), token tile fastest, and each XCD walks a
// contiguous range of them, so the workgroups running at the same time on
// one XCD share a hot expert's weight tile through that XCD's L2.
//
// The plain pass also serves the router GEMM for large batches (one group of
// all T tokens, fp32 out).  There it has only ceil(T/128) x E/WR tiles, so
// with a workspace the K-steps can be split into parts (FfnParams::ksplit):
// item q n + i is part q of tile i, and part q writes its fp32 partial sums
// to its own slice of the output; a second launch adds the parts in order.
#include "moe_kernels.h"

namespace moe {

namespace {

constexpr int BN = 128;  // token rows per tile
constexpr int BK = 64;   // K per step (bf16: 128 bytes per row)
constexpr int ROWB = BK * 2;
constexpr int TOK_BYTES = BN * ROWB;  // 16 KB

typedef __attribute__((address_space(3))) void lds_void;

// 16-byte chunk c (0..7) of LDS row r lives at chunk c ^ (r & 7).
__device__ __forceinline__ int swz(int r, int c) { return r * ROWB + ((c ^ (r & 7)) << 4); }

// One direct-to-LDS load: this lane's 16 bytes at g land at window + 16 *
// lane, window being wave-uniform.
__device__ __forceinline__ void dma16(const uint8_t* g, uint8_t* window) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)window, 16, 0, 0);
}

// s_waitcnt on the vector-memory counter only (expcnt and lgkmcnt at their
// maxima); N < 64.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Workgroup barrier without a memory fence (a fence would wait for every
// load in flight): LDS operations of this wave complete first; the asm
// memory clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

struct TItem {
  int valid, rows0, nrows, K, Nout, f0, m0;
  int s0, S;  // the item's K-steps: [s0, s0 + S)
  const uint8_t* w;
  const uint8_t* act;
  void* out;
};

}  // namespace

template <bool GATED, int WR>
__global__ __launch_bounds__(2 * WR) void gemm_tiled_kernel(FfnParams p) {
  constexpr int NT = 2 * WR;                 // threads: WR / 32 waves
  constexpr int W_BYTES = WR * ROWB;
  constexpr int NWV = NT / 64;
  constexpr int WPW = W_BYTES / 1024 / NWV;    // weight-tile loads per wave and step
  constexpr int TPW = TOK_BYTES / 1024 / NWV;  // token-tile loads per wave and step
  constexpr int P = WPW + TPW;                 // vector-memory ops per wave and step
  // three pipeline stages, each its own array (see the header comment)
  __shared__ __attribute__((aligned(1024))) uint8_t w0[W_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t w1[W_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t w2[W_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t t0[TOK_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t t1[TOK_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t t2[TOK_BYTES];
  __shared__ int s_off[1025];
  __shared__ int s_pre[1025];  // items before active group a
  __shared__ int s_grp[1025];  // expert of active group a
  __shared__ int s_wsum[NT / 64];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int E = p.E;
  // features per item
  constexpr int fcols = GATED ? WR / 2 : WR;
  const int nt_r = p.Nout_r / fcols;
  const int nt_s = p.n_shared ? p.Nout_s / fcols : 0;

  // ---- items per active expert = token tiles x feature tiles; prefix sums
  // compact layout: offsets [E+1]; masked layout: counts [E] (rows of
  // expert e start at e*T)
  for (int e = tid; e <= E; e += NT) s_off[e] = p.masked ? (e < E ? p.expert_offset[e] : 0) : p.expert_offset[e];
  __syncthreads();
  {
    const int per = (E + NT - 1) / NT;
    const int e0 = tid * per;
    int cnt = 0, items = 0;
    for (int i = 0; i < per; ++i) {
      const int e = e0 + i;
      if (e < E) {
        const int n = p.masked ? min(s_off[e], p.T) : s_off[e + 1] - s_off[e];
        if (n > 0) { ++cnt; items += ((n + BN - 1) / BN) * nt_r; }
      }
    }
    // scan (cnt, items) over the block: pack into one 32-bit pair of 16-bit
    // halves would overflow; scan each separately
    int ic = cnt, ii = items;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int yc = __shfl_up(ic, o), yi = __shfl_up(ii, o);
      if (lane >= o) { ic += yc; ii += yi; }
    }
    __shared__ int s_isum[NT / 64];
    if (lane == 63) { s_wsum[wid] = ic; s_isum[wid] = ii; }
    __syncthreads();
    int pc = ic - cnt, pi = ii - items;
    for (int w = 0; w < wid; ++w) { pc += s_wsum[w]; pi += s_isum[w]; }
    for (int i = 0; i < per; ++i) {
      const int e = e0 + i;
      if (e < E) {
        const int n = p.masked ? min(s_off[e], p.T) : s_off[e + 1] - s_off[e];
        if (n > 0) {
          s_grp[pc] = e;
          s_pre[pc] = pi;
          ++pc;
          pi += ((n + BN - 1) / BN) * nt_r;
        }
      }
    }
    if (tid == NT - 1) {
      // totals: one past the last active group holds the routed item count
      s_pre[pc] = pi;
      s_grp[1024] = pc;  // number of active groups
    }
  }
  __syncthreads();
  const int n_active = __builtin_amdgcn_readfirstlane(s_grp[1024]);
  const int routed_items = __builtin_amdgcn_readfirstlane(s_pre[n_active]);
  const int shared_mt = p.n_shared ? (p.T + BN - 1) / BN : 0;
  const int n_items = routed_items + shared_mt * nt_s;
  // split reduction (router GEMM only): item q * n_items + i is part q of tile i
  const int ksp = p.ksplit > 1 ? p.ksplit : 1;

  auto decode = [&](int item_all) {
    TItem it{};
    it.valid = item_all < n_items * ksp;
    if (!it.valid) return it;
    const int part = item_all / n_items, item = item_all - part * n_items;
    int local, mt;
    if (item < routed_items) {
      // binary search: last active group a with s_pre[a] <= item
      int lo = 0, hi = n_active - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_pre[mid] <= item) lo = mid; else hi = mid - 1;
      }
      const int a = __builtin_amdgcn_readfirstlane(lo);
      const int g = __builtin_amdgcn_readfirstlane(s_grp[a]);
      local = item - __builtin_amdgcn_readfirstlane(s_pre[a]);
      it.rows0 = p.masked ? g * p.T : __builtin_amdgcn_readfirstlane(s_off[g]);
      it.nrows = p.masked ? min(__builtin_amdgcn_readfirstlane(s_off[g]), p.T)
                          : __builtin_amdgcn_readfirstlane(s_off[g + 1]) - it.rows0;
      mt = (it.nrows + BN - 1) / BN;
      it.K = p.K_r;
      it.Nout = p.Nout_r;
      it.w = p.w + (size_t)g * p.NW_r * p.K_r * 2;
      it.act = p.act;
      it.out = p.out;
    } else {
      local = item - routed_items;
      it.rows0 = 0;
      it.nrows = p.T;
      mt = shared_mt;
      it.K = p.K_s;
      it.Nout = p.Nout_s;
      it.w = p.s_w;
      it.act = p.s_act;
      it.out = p.s_out;
    }
    // token tile fastest: consecutive items share one weight tile
    it.m0 = (local % mt) * BN;
    it.f0 = (local / mt) * fcols;
    const int steps = it.K / BK;
    it.s0 = part * steps / ksp;
    it.S = (part + 1) * steps / ksp - it.s0;
    if (ksp > 1) it.out = static_cast<float*>(it.out) + (size_t)part * p.T * it.Nout;
    return it;
  };

  // Direct-to-LDS loads: load q of wave w fills LDS rows r0 = 8 (w WPW + q)
  // .. r0 + 7 of the weight tile (likewise for the token tile); lane l
  // fetches row r0 + l / 8, chunk (l % 8) ^ (l / 8), which lands at chunk
  // position l % 8 of that row, i.e. swizzled as swz() expects.
  const int lsub = lane >> 3, lchunk = ((lane & 7) ^ lsub) << 4;
  const uint8_t* gw[WPW];
  const uint8_t* gt[TPW];
  auto set_rows = [&](const TItem& it) {
    const size_t rowbytes = (size_t)it.K * 2;
#pragma unroll
    for (int q = 0; q < WPW; ++q) {
      const int lr = 8 * (wid * WPW + q) + lsub;
      int wr;
      if (GATED) wr = lr < WR / 2 ? it.f0 + lr : it.Nout + it.f0 + (lr - WR / 2);
      else wr = it.f0 + lr;
      gw[q] = it.w + (size_t)wr * rowbytes + lchunk;
    }
#pragma unroll
    for (int q = 0; q < TPW; ++q) {
      int tr = it.m0 + 8 * (wid * TPW + q) + lsub;
      tr = tr < it.nrows ? tr : 0;  // rows past the group: never stored
      gt[q] = it.act + (size_t)(it.rows0 + tr) * rowbytes + lchunk;
    }
  };
  // Steps past the end load one line of the expert's weights instead (never
  // read), so that every step issues exactly P loads and the wait counts
  // below hold on every path.
  auto issue = [&](const TItem& it, int s, int S, uint8_t* wb, uint8_t* tb) {
    const bool real = s < S;
    const size_t kb = (size_t)(it.s0 + s) * ROWB;
#pragma unroll
    for (int q = 0; q < WPW; ++q) dma16(real ? gw[q] + kb : it.w, wb + 1024 * (wid * WPW + q));
#pragma unroll
    for (int q = 0; q < TPW; ++q) dma16(real ? gt[q] + kb : it.w, tb + 1024 * (wid * TPW + q));
  };

  // wave block: weight rows (4 blocks of 16) x token rows (4 blocks of 16)
  const int wn = wid >> 1, wm = wid & 1;
  int arow[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    if (GATED) arow[nb] = (nb < 2 ? 0 : WR / 2) + 32 * wn + 16 * (nb & 1);
    else arow[nb] = 64 * wn + 16 * nb;
  }
  const int brow0 = 64 * wm;
  const int g4 = lane >> 4, r16 = lane & 15;

  f32x4_t acc[4][4];
  // Both 32-wide sub-steps' operands are read up front.  The schedule (group
  // barriers below): the first sub-step's eight reads, then the step's
  // direct-to-LDS loads, then its MFMAs with the second sub-step's reads
  // slotted between them, then the rest; so the MFMA pipe waits for LDS only
  // once per step, right after the barrier.
  auto compute = [&](const uint8_t* wb, const uint8_t* tb) {
    bf16x8_t av[2][4], bv[2][4];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int ch = 4 * ks + g4;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        av[ks][nb] = *reinterpret_cast<const bf16x8_t*>(wb + swz(arow[nb] + r16, ch));
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        bv[ks][mb] = *reinterpret_cast<const bf16x8_t*>(tb + swz(brow0 + 16 * mb + r16, ch));
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[ks][nb], bv[ks][mb], acc[nb][mb], 0, 0, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);  // LDS reads
    __builtin_amdgcn_sched_group_barrier(0x020, P, 0);  // direct-to-LDS loads
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 24, 0);
  };

  auto epilogue = [&](const TItem& it) {
    const int Nout = it.Nout;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int tok = it.m0 + brow0 + 16 * mb + r16;
      if (tok >= it.nrows) continue;
      const size_t r = (size_t)(it.rows0 + tok);
      if constexpr (GATED) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const int f = it.f0 + 32 * wn + 16 * nb + 4 * g4;
          float h[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) h[j] = silu(acc[nb][mb][j]) * acc[nb + 2][mb][j];
          const uint32_t lo = f32_to_bf16_bits(h[0]) | (f32_to_bf16_bits(h[1]) << 16);
          const uint32_t hi = f32_to_bf16_bits(h[2]) | (f32_to_bf16_bits(h[3]) << 16);
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(it.out) + r * Nout + f) = make_uint2(lo, hi);
        }
      } else {
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const int f = it.f0 + 64 * wn + 16 * nb + 4 * g4;
          *reinterpret_cast<f32x4_t*>(static_cast<float*>(it.out) + r * Nout + f) = acc[nb][mb];
        }
      }
    }
  };

  // XCD-contiguous walk: workgroup b runs on XCD b % 8; each XCD takes a
  // contiguous eighth of the items, so its concurrently running workgroups
  // cover consecutive items (the token tiles of one weight tile) and share
  // the weight tile through that XCD's L2.  Measured against a plain stride
  // with feature tiles fastest: 4096-token prefill down pass 2203 -> 2107 us,
  // 128 experts x 32 rows gate/up 201 -> 168 us.
  const int nx = gridDim.x % 8 == 0 ? 8 : 1;
  const int xcd = blockIdx.x % nx, slot = blockIdx.x / nx;
  const int per_x = gridDim.x / nx;
  const int n_all = n_items * ksp;
  const int span = (n_all + nx - 1) / nx;
  const int lo_x = xcd * span, hi_x = min(n_all, lo_x + span);
  for (int item = lo_x + slot; item < hi_x; item += per_x) {
    const TItem it = decode(item);
    const int S = it.S;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) acc[nb][mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    set_rows(it);
    // Pipeline: steps st+1 and st+2 are landing while step st is multiplied
    // out of LDS.  Step st lives in stage st % 3; the loop is unrolled by
    // three so that every access names its stage array directly.  Loads,
    // waits and barriers run for a whole number of three-step rounds on
    // every wave; only the MFMAs of steps past the end are skipped.
    issue(it, 0, S, w0, t0);
    issue(it, 1, S, w1, t1);
    auto step = [&](int st, uint8_t* wb, uint8_t* tb, uint8_t* wn2, uint8_t* tn2) {
      // this wave's loads of step st are done when only the P loads of step
      // st+1 remain; every wave's are, after the barrier, which also frees
      // stage (st+2) % 3 (read at step st-1)
      wait_vm<P>();
      lds_barrier();
      issue(it, st + 2, S, wn2, tn2);
      if (st < S) compute(wb, tb);
    };
    const int S3 = (S + 2) / 3 * 3;
    for (int s = 0; s < S3; s += 3) {
      step(s, w0, t0, w2, t2);
      step(s + 1, w1, t1, w0, t0);
      step(s + 2, w2, t2, w1, t1);
    }
    wait_vm<0>();  // the last two steps' placeholder loads
    epilogue(it);
    lds_barrier();  // the stages are refilled by the next item
  }
}

template <bool GATED, int WR>
static hipError_t launch_wr(const FfnParams& p, long long max_token_tiles, hipStream_t stream) {
  constexpr int fcols = GATED ? WR / 2 : WR;
  const long long max_items = (max_token_tiles * (p.Nout_r / fcols) +
                               (p.n_shared ? (long long)((p.T + BN - 1) / BN) * (p.Nout_s / fcols) : 0)) *
                              (p.ksplit > 1 ? p.ksplit : 1);
  auto kern = gemm_tiled_kernel<GATED, WR>;
  // constant per kernel and device model: computed once (thread-safe
  // initialisation of a const local static)
  static const Residency occ = [&] {
    Residency o{};
    int dev = 0, n = 0, c = 0;
    if (hipGetDevice(&dev) != hipSuccess) return o;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, 2 * WR, 0) != hipSuccess) n = 1;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) c = 256;
    o.per_cu = n > 0 ? n : 1;
    o.cus = c;
    o.ok = true;
    return o;
  }();
  if (!occ.ok) return hipErrorInvalidDevice;
  const long long cap = (long long)occ.per_cu * occ.cus;
  const int grid = (int)(max_items < cap ? max_items : cap);
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(2 * WR), 0, stream, p);
  return hipGetLastError();
}

// Weight rows per tile: 256 (128 features) in the gated pass, whose output
// count is a multiple of 128 for every accepted configuration; in the plain
// pass 256 when every group's output count is a multiple of 256, else 128.
hipError_t launch_gemm_tiled(const FfnParams& p, bool gated, long long max_token_tiles, hipStream_t stream) {
  if (gated) return launch_wr<true, 256>(p, max_token_tiles, stream);
  if (p.Nout_r % 256 == 0 && (!p.n_shared || p.Nout_s % 256 == 0))
    return launch_wr<false, 256>(p, max_token_tiles, stream);
  return launch_wr<false, 128>(p, max_token_tiles, stream);
}

}  // namespace moe
