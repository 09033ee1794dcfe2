// Grouped expert GEMMs for prefill-sized batches (bf16).  "7.13 Serving
// Mixture-of-Experts", section "Prefill vs. Decode": with many tokens per
// expert the grouped GEMM is fat and each weight tile can be reused across
// many token rows.
//
// Design (gfx950): work item = (group, 128-row token tile, feature tile).
// A workgroup of WR/32 waves computes a WR x 128 block: WR weight rows (the
// gate and up rows of WR/2 features in the gated pass, WR output features in
// the plain pass) against 128 token rows, K in steps of 64.  Each step's tiles go
// HBM -> registers (three steps in flight) -> LDS (double buffered, 16-byte
// chunks XOR-swizzled by row so the MFMA operand reads are free of bank
// conflicts).  Each wave owns a 64 x 64 block (4 x 4 MFMA tiles) and, in the
// gated pass, holds matching gate and up columns, so SwiGLU is applied in
// registers (MFMA: v_mfma_f32_16x16x32_bf16).  WR = 256 when the feature
// count allows: one token tile then feeds twice as many weight rows.  Items
// are ordered (group, token tile, feature tile), feature tile fastest, so
// the workgroups running at the same time share token tiles and the hot
// experts' weight tiles through the L2 and the Infinity Cache.
//
// Measured limit: a CU's L1 keeps a bounded number of L2 requests in flight,
// so at this tile size (48 KB of operands per K step for 4.2 MFLOP) the
// kernel is bound by the L2 -> CU path, not by MFMA issue; the prefill layer
// is in any case bounded below by streaming each touched expert's weights
// from HBM once.
#include "moe_kernels.h"

namespace moe {

namespace {

constexpr int BN = 128;  // token rows per tile
constexpr int BK = 64;   // K per step (bf16: 128 bytes per row)
constexpr int ROWB = BK * 2;
constexpr int TOK_BYTES = BN * ROWB;  // 16 KB

template <int TQ>
struct Chunk {
  i32x4_t a[4];   // this thread's 64 bytes of the weight tile
  i32x4_t b[TQ];  // and its TQ * 16 bytes of the token tile
};

// 16-byte chunk c (0..7) of LDS row r lives at chunk c ^ (r & 7).
__device__ __forceinline__ int swz(int r, int c) { return r * ROWB + ((c ^ (r & 7)) << 4); }

struct TItem {
  int valid, rows0, nrows, K, Nout, f0, m0;
  const uint8_t* w;
  const uint8_t* act;
  void* out;
};

}  // namespace

template <bool GATED, int WR>
__global__ __launch_bounds__(2 * WR) void gemm_tiled_kernel(FfnParams p) {
  constexpr int NT = 2 * WR;                 // threads: WR / 32 waves
  constexpr int W_BYTES = WR * ROWB;
  constexpr int TQ = TOK_BYTES / NT / 16;    // token 16-byte chunks per thread
  constexpr int TPR = ROWB / (16 * TQ);      // threads per token row
  __shared__ __attribute__((aligned(16))) uint8_t lds_w[2][W_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t lds_t[2][TOK_BYTES];
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
  for (int e = tid; e <= E; e += NT) s_off[e] = p.expert_offset[e];
  __syncthreads();
  {
    const int per = (E + NT - 1) / NT;
    const int e0 = tid * per;
    int cnt = 0, items = 0;
    for (int i = 0; i < per; ++i) {
      const int e = e0 + i;
      if (e < E) {
        const int n = s_off[e + 1] - s_off[e];
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
        const int n = s_off[e + 1] - s_off[e];
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

  auto decode = [&](int item) {
    TItem it{};
    it.valid = item < n_items;
    if (!it.valid) return it;
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
      it.rows0 = __builtin_amdgcn_readfirstlane(s_off[g]);
      it.nrows = __builtin_amdgcn_readfirstlane(s_off[g + 1]) - it.rows0;
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
    // feature tile fastest: consecutive items share one token tile
    const int nt = item < routed_items ? nt_r : nt_s;
    it.f0 = (local % nt) * fcols;
    it.m0 = (local / nt) * BN;
    (void)mt;
    return it;
  };

  // global -> registers: thread t owns weight row t/2, bytes [64 (t&1), +64),
  // and token row t / TPR, bytes [16 TQ (t % TPR), +16 TQ)
  const int lrow = tid >> 1, lhalf = tid & 1;
  const int trow = tid / TPR, tchunk = (tid % TPR) * TQ;
  auto gload = [&](Chunk<TQ>& c, const TItem& it, int s) {
    const size_t rowbytes = (size_t)it.K * 2;
    const size_t kb = (size_t)s * ROWB;
    int wr;
    if (GATED) wr = lrow < WR / 2 ? it.f0 + lrow : it.Nout + it.f0 + (lrow - WR / 2);
    else wr = it.f0 + lrow;
    const uint8_t* pa = it.w + (size_t)wr * rowbytes + kb + 64 * lhalf;
    int tr = it.m0 + trow;
    tr = tr < it.nrows ? tr : 0;  // rows past the group: never stored
    const uint8_t* pb = it.act + (size_t)(it.rows0 + tr) * rowbytes + kb + 16 * tchunk;
#pragma unroll
    for (int q = 0; q < 4; ++q) c.a[q] = *reinterpret_cast<const i32x4_t*>(pa + 16 * q);
#pragma unroll
    for (int q = 0; q < TQ; ++q) c.b[q] = *reinterpret_cast<const i32x4_t*>(pb + 16 * q);
  };
  auto lstore = [&](const Chunk<TQ>& c, int buf) {
#pragma unroll
    for (int q = 0; q < 4; ++q) *reinterpret_cast<i32x4_t*>(&lds_w[buf][swz(lrow, 4 * lhalf + q)]) = c.a[q];
#pragma unroll
    for (int q = 0; q < TQ; ++q) *reinterpret_cast<i32x4_t*>(&lds_t[buf][swz(trow, tchunk + q)]) = c.b[q];
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
  auto compute = [&](int buf) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int ch = 4 * ks + g4;
      bf16x8_t av[4], bv[4];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        av[nb] = *reinterpret_cast<const bf16x8_t*>(&lds_w[buf][swz(arow[nb] + r16, ch)]);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        bv[mb] = *reinterpret_cast<const bf16x8_t*>(&lds_t[buf][swz(brow0 + 16 * mb + r16, ch)]);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[nb], bv[mb], acc[nb][mb], 0, 0, 0);
    }
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

  // Plain stride over the items: the workgroups that run together cover a
  // window of consecutive items (spread over all XCDs, sharing through the
  // Infinity Cache), which measured faster than giving each XCD a contiguous
  // range of its own.
  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const TItem it = decode(item);
    const int S = it.K / BK;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) acc[nb][mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // Pipeline: registers hold steps s+1..s+3 while step s is multiplied out
    // of LDS.  Steps past the end reload the last step (never used).
    Chunk<TQ> rg[3];
    auto cl = [&](int s) { return s < S ? s : S - 1; };
    gload(rg[0], it, 0);
    gload(rg[1], it, cl(1));
    gload(rg[2], it, cl(2));
    // step 0 into LDS buffer 0
    lstore(rg[0], 0);
    __syncthreads();
    gload(rg[0], it, cl(3));
    // Three steps per iteration (compile-time register slots).  Loads,
    // stores and barriers run unconditionally so that every wave meets the
    // same barriers and the compiler's wait counts stay exact; only the
    // MFMAs of steps past the end are skipped.
    const int S3 = (S + 2) / 3 * 3;
    for (int s = 0; s < S3; s += 3) {
#pragma unroll
      for (int r = 0; r < 3; ++r) {
        const int st = s + r;
        if (st < S) compute(st & 1);
        // step st+1 (slot (r+1)%3) goes to the other buffer
        lstore(rg[(r + 1) % 3], (st + 1) & 1);
        __syncthreads();
        // refill the slot just stored with step st+4
        gload(rg[(r + 1) % 3], it, cl(st + 4));
      }
    }
    epilogue(it);
    __syncthreads();  // LDS buffers are reused by the next item
  }
}

template <bool GATED, int WR>
static hipError_t launch_wr(const FfnParams& p, long long max_token_tiles, hipStream_t stream) {
  constexpr int fcols = GATED ? WR / 2 : WR;
  const long long max_items = max_token_tiles * (p.Nout_r / fcols) +
                              (p.n_shared ? (long long)((p.T + BN - 1) / BN) * (p.Nout_s / fcols) : 0);
  auto kern = gemm_tiled_kernel<GATED, WR>;
  static int per_cu = -1, cus = -1;  // constant per kernel and device model
  if (per_cu < 0) {
    int dev = 0, n = 0, c = 0;
    if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, 2 * WR, 0) != hipSuccess) n = 1;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) c = 256;
    per_cu = n > 0 ? n : 1;
    cus = c;
  }
  const long long cap = (long long)per_cu * cus;
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
