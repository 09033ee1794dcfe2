// Grouped expert GEMMs over the dispatch buffer (read in place) and the shared
// expert, for decode-sized batches.  "7.13 Serving Mixture-of-Experts",
// section "Expert Parallelism Mechanics", step 3: one grouped GEMM runs all
// local experts' matmuls in a single launch; section "Prefill vs. Decode": at
// decode each expert sees a handful of rows, so the pass is bound by streaming
// the touched experts' weights from HBM.
//
// Design (gfx950):
//  * The weights are the MFMA A operand and go straight from HBM into
//    registers: each step a wave reads 256 bytes of each of its 16 rows.  The
//    activation rows (one 16-token tile per MFMA column block) are the B
//    operand.  Experts with no rows own no work, so their weights are never
//    read.
//  * Work item = (group, 16-row chunk of the group's rows, tile of 16*FW
//    output columns).  Groups are the experts that received rows, in index
//    order, then the shared expert.  Every chunk is an item of its own, so a
//    group with many rows (the shared expert sees all T tokens) is spread
//    over many workgroups that stream the same weights at about the same
//    time, instead of one workgroup walking K once per chunk.  A workgroup
//    has FW x KS waves: FW column tiles, each reduction dimension split KS
//    ways; the KS partial sums are added through LDS in a fixed order
//    (results do not depend on timing or slot order).
//  * Workgroups are persistent: workgroup b of n walks items b, b + n, ...
//    and every wave streams its sequence of (item, K-step) stages through a
//    three-slot register ring, two stages ahead, across item boundaries, so
//    loads stay in flight while an item's epilogue runs.
//    Loads are never skipped (a stage past the end repeats the last address,
//    a token row past a group's end reads the group's first row and its
//    column is never stored), which keeps the wait counts exact.
//  * A CU takes in only so many bytes per microsecond when its loads mix HBM
//    misses with L2 hits, and every column wave needs the same activation
//    tile at a step.  Where the waves of a workgroup walk the same steps,
//    they share that tile through LDS (SHARE, below) instead of each loading
//    it; the launch plan (launch_ffn) picks the shape per pass from the
//    K-steps per item and the rows per touched expert.
//  * The same walk, with one group holding all T tokens and fp32 output, is
//    the router GEMM for 17-2047 tokens (launch_router_gemm).
#include "route_body.h"

namespace moe {

__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

// One pipeline stage of a wave: NMAT weight tiles and the activation tiles
// they multiply (NX = 1: every weight tile walks K in the same order).  With
// a shared activation tile (XP > 0) the wave holds only its XP 16-byte pieces
// of the tile, on their way to LDS, and x is unused.
template <int DT, int NMAT, int TT, int NX, int XP = 0>
struct Stage {
  Step w[NMAT];
  Step x[NX][TT];
  i32x4_t xp[XP > 0 ? XP : 1];
  float sx[NX][TT][2]; // E4M3 activation scales of the step's two 128-blocks
  float sw[NMAT][2];   // E4M3 weight block scales of the step
};

// Everything about one item that the loads and the epilogue need; all fields
// are uniform across the wave.
struct Item {
  int valid;
  int rows0, nrows, K, Nout, col0, s_begin, s_end, rot;
  const uint8_t* w;
  const uint8_t* act;
  const float* act_scale;
  const float* w_scale;
  void* out;
  float* out_scale;
};

struct Cursor {
  Item it;
  int item, step;
};

template <int DT, int FW, int KS, int TT, int WC>
struct Walker {
  static constexpr int ES = Elem<DT>::kBytes;
  static constexpr int STEP = Elem<DT>::kStep;
  const FfnParams& p;
  const int* s_off;
  const int* s_act;
  const int* s_pre;  // items before active group a; s_pre[n_active] = routed items
  int n_active, n_routed_items, n_items, ft, kp, nblk;
  bool single;  // every active group is one chunk: group a owns items [a tiles_r, (a+1) tiles_r)

  __device__ Item decode(int item) const {
    Item it{};
    it.valid = item < n_items;
    if (!it.valid) return it;
    int tile, chunk, K, rows0, nrows, key;
    if (item < n_routed_items) {
      // last active group a with s_pre[a] <= item
      int lo, local;
      if (single) {
        lo = item / p.tiles_r;
        local = item - lo * p.tiles_r;
      } else {
        lo = 0;
        int hi = n_active - 1;
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (s_pre[mid] <= item) lo = mid; else hi = mid - 1;
        }
        local = item - uni(s_pre[lo]);
      }
      const int a = uni(lo);
      chunk = local / p.tiles_r;
      tile = local - chunk * p.tiles_r;
      const int g = uni(s_act[a]);
      key = g * p.tiles_r + tile;
      rows0 = p.masked ? g * p.T : uni(s_off[g]);
      nrows = p.masked ? uni(s_off[g]) : uni(s_off[g + 1]) - rows0;
      K = p.K_r;
      it.Nout = p.Nout_r;
      it.w = p.w + (size_t)g * p.NW_r * K * ES;
      it.act = p.act;
      it.act_scale = p.act_scale;
      it.w_scale = p.w_scale ? p.w_scale + (size_t)g * (p.NW_r / 128) * (K / 128) : nullptr;
      it.out = p.out;
      it.out_scale = p.out_scale;
    } else {
      const int local = item - n_routed_items;
      chunk = local / p.tiles_s;
      tile = local - chunk * p.tiles_s;
      key = (1 << 20) + tile;  // independent of E: the same whichever launch runs it
      rows0 = 0;
      nrows = p.T;
      K = p.K_s;
      it.Nout = p.Nout_s;
      it.w = p.s_w;
      it.act = p.s_act;
      it.act_scale = p.s_act_scale;
      it.w_scale = p.s_w_scale;
      it.out = p.s_out;
      it.out_scale = p.s_out_scale;
    }
    it.K = K;
    it.col0 = tile * WC * FW + ft * WC;
    it.rows0 = rows0 + chunk * TT * 16;
    it.nrows = min(TT * 16, nrows - chunk * TT * 16);
    const int steps = K / STEP;
    it.s_begin = kp * steps / KS;
    it.s_end = (kp + 1) * steps / KS;
    // Items start their K walk at different offsets: waves that run in
    // lockstep then touch different DRAM channels even when rows are a
    // multiple of the channel interleave apart.  The offset is a function of
    // (group, column tile) only, so every row of a group is summed in the
    // same order whichever chunk its dispatch slot falls in.
    it.rot = (int)(((unsigned)key * 2654435761u) >> 16) % (it.s_end - it.s_begin);
    return it;
  }

  // K-step actually read at logical position `step` of an item
  __device__ int phys(const Cursor& c) const {
    int s = c.step - c.it.s_begin + c.it.rot;
    const int n = c.it.s_end - c.it.s_begin;
    if (s >= n) s -= n;
    return c.it.s_begin + s;
  }

  __device__ void start(Cursor& c, int item) const {
    c.item = item;
    c.it = decode(item);
    c.step = c.it.s_begin;
  }

  // Next stage; past the last one the cursor stays put (it.valid stays 1 for
  // the issue cursor so its loads keep a valid address) and *done is set.
  __device__ void advance(Cursor& c, bool& done) const {
    if (++c.step < c.it.s_end) return;
    const Item nx = decode(c.item + nblk);
    if (!nx.valid) {
      done = true;
      c.step = c.it.s_end - 1;
      return;
    }
    c.item += nblk;
    c.it = nx;
    c.step = c.it.s_begin;
  }
};

// Workgroup barrier that orders LDS only: the wave's LDS operations complete,
// then s_barrier.  __syncthreads() would also wait for every global load in
// flight, which would drain the streaming ring at every step.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// NM: 16-row weight tiles a wave streams together: the gate and up tiles of
// the same 16 columns (gated pass), or NM adjacent 16-column tiles (plain).
//
// SHARE: the FW waves that walk the same K-steps (same kp) share each step's
// activation tile through LDS instead of each loading all of it: every lane
// loads XP pieces of PB bytes (16, or 8 when the tile has fewer 16-byte
// pieces than the waves have lanes), writes them to one of three LDS slots a
// stage ahead, and after one LDS-only barrier per stage all FW waves read
// their MFMA B operands from the slot.  Needs the same number of K-steps per
// item on every wave (the launch checks that the K-split divides every
// item's steps), so that all waves of the workgroup meet the same barriers
// in the same order.
template <int DT, int FW, int KS, int TT, bool GATED, int OUT, int NM, bool PARK = true, bool SHARE = false>
__device__ __forceinline__ void ffn_body(const FfnParams& p, int bid, int nblk) {
  constexpr int NMAT = GATED ? 2 : NM;
  constexpr int NX = 1;                     // activation tiles per stage
  constexpr int WC = GATED ? 16 : 16 * NM;  // output columns per wave
  constexpr int NT = 64 * FW * KS;
  constexpr bool FP8 = DT == MOE_FP8_E4M3;
  constexpr int RED = (KS > 1 ? (KS - 1) : 1) * FW * NMAT * TT * 4 * 64;
  constexpr int XT = TT * 16 * 256;  // bytes of one step's activation tile
  constexpr int PB = XT % (64 * FW * 16) == 0 ? 16 : 8;  // bytes per piece
  constexpr int PPR = 256 / PB;                           // pieces per tile row
  constexpr int XP = SHARE ? XT / (64 * FW * PB) : 0;     // pieces per lane
  static_assert(!SHARE || (XP >= 1 && XP * 64 * FW * PB == XT), "shared activation tiles");
  using W = Walker<DT, FW, KS, TT, WC>;
  using St = Stage<DT, NMAT, TT, NX, XP>;
  __shared__ float red[RED];
  // three stage slots per K-split part, rows XOR-swizzled in 16-byte units
  __shared__ __attribute__((aligned(16))) uint8_t xs[SHARE ? 3 * KS * XT : 16];
  __shared__ float amax_s[FW][TT * 16];
  __shared__ int s_off[1025];
  __shared__ int s_act[1024];
  __shared__ int s_pre[1025];
  __shared__ int s_wsum[NT / 64];
  __shared__ int s_isum[NT / 64];

  const int tid = threadIdx.x;
  // wave-uniform values go through readfirstlane so that everything derived
  // from them (item decode, loop bounds) stays in scalar registers and the
  // loop needs no vector waits beyond the ring's own loads
  const int lane = tid & 63, wid = uni(tid >> 6);
  const int ft = wid % FW, kp = wid / FW;
  const int E = p.E;

  // ---- experts with rows, in index order, and the items before each
  // (chunks x tiles), once per workgroup
  // compact layout: offsets [E+1]; masked layout: counts [E] (rows of
  // expert e start at e*T)
  for (int e = tid; e <= E; e += NT) s_off[e] = p.masked ? (e < E ? p.expert_offset[e] : 0) : p.expert_offset[e];
  __syncthreads();
  constexpr int CH = TT * 16;  // rows per chunk
  {
    const int per = (E + NT - 1) / NT;
    const int e0 = tid * per;
    int cnt = 0, items = 0;
    for (int i = 0; i < per; ++i) {
      const int e = e0 + i;
      if (e < E) {
        const int n = p.masked ? s_off[e] : s_off[e + 1] - s_off[e];
        if (n > 0) { ++cnt; items += (n + CH - 1) / CH * p.tiles_r; }
      }
    }
    int ic = cnt, ii = items;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int yc = __shfl_up(ic, o), yi = __shfl_up(ii, o);
      if (lane >= o) { ic += yc; ii += yi; }
    }
    if (lane == 63) { s_wsum[wid] = ic; s_isum[wid] = ii; }
    __syncthreads();
    int pc = ic - cnt, pi = ii - items;
    for (int w = 0; w < wid; ++w) { pc += s_wsum[w]; pi += s_isum[w]; }
    for (int i = 0; i < per; ++i) {
      const int e = e0 + i;
      if (e < E) {
        const int n = p.masked ? s_off[e] : s_off[e + 1] - s_off[e];
        if (n > 0) {
          s_act[pc] = e;
          s_pre[pc] = pi;
          ++pc;
          pi += (n + CH - 1) / CH * p.tiles_r;
        }
      }
    }
    if (tid == NT - 1) s_pre[pc] = pi;  // total routed items after the last group
  }
  int n_active = 0;
  for (int w = 0; w < NT / 64; ++w) n_active += s_wsum[w];
  n_active = uni(n_active);
  __syncthreads();
  const int routed_items = uni(s_pre[n_active]);
  const int shared_items = p.n_shared ? (p.T + CH - 1) / CH * p.tiles_s : 0;

  const W walk{p, s_off, s_act, s_pre, n_active, routed_items, routed_items + shared_items, ft, kp, nblk,
               routed_items == n_active * p.tiles_r};
  if (bid >= walk.n_items) return;  // uniform per block

  const int r16 = lane & 15;
  // piece i of this lane covers bytes [(i % PPR) PB, +PB) of tile row i / PPR
  auto piece = [&](int q) { return (q * FW + ft) * 64 + lane; };
  auto load = [&](St& s, const Cursor& c) {
    const size_t rowbytes = (size_t)c.it.K * W::ES;
    if constexpr (SHARE) {
      // issued first: the LDS write a stage later then waits only for these
      const int ps = walk.phys(c);
#pragma unroll
      for (int q = 0; q < XP; ++q) {
        const int i = piece(q);
        int row = i / PPR;
        row = row < c.it.nrows ? row : 0;  // rows past the group's end: never stored
        const uint8_t* src = c.it.act + (size_t)(c.it.rows0 + row) * rowbytes + (size_t)ps * 256 + (i % PPR) * PB;
        if constexpr (PB == 16) {
          s.xp[q] = *reinterpret_cast<const i32x4_t*>(src);
        } else {
          const uint2 v = *reinterpret_cast<const uint2*>(src);
          s.xp[q] = i32x4_t{(int)v.x, (int)v.y, 0, 0};
        }
      }
    }
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
      const int ps = walk.phys(c);
      const int row = (GATED ? (m == 0 ? 0 : c.it.Nout) : 16 * m) + c.it.col0 + r16;
      load_step(s.w[m], c.it.w + (size_t)row * rowbytes + (size_t)ps * 256, lane);
      if constexpr (FP8) {
        const int wsrow = ((GATED ? (m == 0 ? 0 : c.it.Nout) : 16 * m) + c.it.col0) / 128;
        const float* wsp = c.it.w_scale + (size_t)wsrow * (c.it.K / 128) + 2 * ps;
        s.sw[m][0] = wsp[0];
        s.sw[m][1] = wsp[1];
      }
    }
#pragma unroll
    for (int xi = 0; xi < NX; ++xi) {
      const int ps = walk.phys(c);
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        int col = tt * 16 + r16;
        col = col < c.it.nrows ? col : 0;  // rows past the group's end: never stored
        const size_t row = (size_t)(c.it.rows0 + col);
        if constexpr (!SHARE) load_step(s.x[xi][tt], c.it.act + row * rowbytes + (size_t)ps * 256, lane);
        if constexpr (FP8) {
          const float* sp = c.it.act_scale + row * (c.it.K / 128) + 2 * ps;
          s.sx[xi][tt][0] = sp[0];
          s.sx[xi][tt][1] = sp[1];
        }
      }
    }
  };

  f32x4_t acc[NMAT][TT];
  auto zero_acc = [&]() {
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) acc[m][tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  };

  // this lane's pieces of a stage -> LDS slot
  auto put = [&](const St& s, int slot) {
    if constexpr (SHARE) {
      uint8_t* base = xs + (slot * KS + kp) * XT;
#pragma unroll
      for (int q = 0; q < XP; ++q) {
        const int i = piece(q), row = i / PPR, b = (i % PPR) * PB;
        uint8_t* dst = base + row * 256 + ((((b >> 4) ^ (row & 15)) << 4) | (b & 15));
        if constexpr (PB == 16) *reinterpret_cast<i32x4_t*>(dst) = s.xp[q];
        else *reinterpret_cast<uint2*>(dst) = make_uint2((unsigned)s.xp[q][0], (unsigned)s.xp[q][1]);
      }
    }
  };
  // activation operand of token tile tt: from the stage, or from LDS slot
  auto xstep = [&](const St& s, int slot, int tt) {
    if constexpr (SHARE) {
      Step b;
      const uint8_t* base = xs + (slot * KS + kp) * XT;
      const int row = tt * 16 + r16, g = lane >> 4;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        b.q[q] = *reinterpret_cast<const i32x4_t*>(base + row * 256 + (((4 * q + g) ^ (row & 15)) << 4));
      return b;
    } else {
      return s.x[0][tt];
    }
  };
  auto compute = [&](const St& s, const Cursor& c, int slot) {
    const int left = c.it.nrows;  // rows of this item (> 0)
    Step xb[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
      if (SHARE && tt * 16 < left) xb[tt] = xstep(s, slot, tt);
    if constexpr (FP8) {
#pragma unroll
      for (int m = 0; m < NMAT; ++m) {
        const float sw0 = s.sw[m][0], sw1 = s.sw[m][1];
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
          if (tt * 16 < left) {
            const int xi = 0;
            const Step& xv = SHARE ? xb[tt] : s.x[xi][tt];
            const f32x4_t p0 = mma_fp8_block(s.w[m], xv, 0);
            const f32x4_t p1 = mma_fp8_block(s.w[m], xv, 1);
            const float c0 = sw0 * s.sx[xi][tt][0], c1 = sw1 * s.sx[xi][tt][1];
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[m][tt][j] += p0[j] * c0 + p1[j] * c1;
          }
        }
      }
    } else {
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
          if (tt * 16 < left) Mma<DT>::run(acc[m][tt], s.w[m], SHARE ? xb[tt] : s.x[0][tt]);
    }
  };

  // End of an item: add the KS partial sums, apply the epilogue.
  auto finish = [&](f32x4_t (&acc)[NMAT][TT], const Cursor& c) {
    if constexpr (KS > 1) {
      if (kp > 0) {
        float* dst = red + ((size_t)((kp - 1) * FW + ft) * NMAT * TT * 4) * 64;
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
          for (int tt = 0; tt < TT; ++tt)
#pragma unroll
            for (int j = 0; j < 4; ++j) dst[((m * TT + tt) * 4 + j) * 64 + lane] = acc[m][tt][j];
      }
      __syncthreads();
      if (kp == 0) {
        for (int q = 1; q < KS; ++q) {
          const float* src = red + ((size_t)((q - 1) * FW + ft) * NMAT * TT * 4) * 64;
#pragma unroll
          for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int tt = 0; tt < TT; ++tt)
#pragma unroll
              for (int j = 0; j < 4; ++j) acc[m][tt][j] += src[((m * TT + tt) * 4 + j) * 64 + lane];
        }
      }
    }
    // lane holds output columns col0 + 4 (lane/16) + j of the item's row tt*16 + lane%16
    const int cfirst = c.it.col0 + 4 * (lane >> 4);
    const int Nout = c.it.Nout;
    if constexpr (GATED) {
      float h[TT][4];
#pragma unroll
      for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int j = 0; j < 4; ++j) h[tt][j] = silu(acc[0][tt][j]) * acc[1][tt][j];
      if constexpr (OUT == MOE_FP8_E4M3) {
        // per-token amax over the item's 128 columns, then E4M3 codes
        if (kp == 0) {
#pragma unroll
          for (int tt = 0; tt < TT; ++tt) {
            float a = fmaxf(fmaxf(fabsf(h[tt][0]), fabsf(h[tt][1])), fmaxf(fabsf(h[tt][2]), fabsf(h[tt][3])));
            a = fmaxf(a, __shfl_xor(a, 16));
            a = fmaxf(a, __shfl_xor(a, 32));
            if (lane < 16) amax_s[ft][tt * 16 + lane] = a;
          }
        }
        __syncthreads();
        if (kp == 0) {
#pragma unroll
          for (int tt = 0; tt < TT; ++tt) {
            const int col = tt * 16 + r16;
            if (col < c.it.nrows) {
              float a = 0.f;
#pragma unroll
              for (int f = 0; f < FW; ++f) a = fmaxf(a, amax_s[f][tt * 16 + r16]);
              const float scale = a > 0.f ? a / 448.0f : 1.0f;
              uint32_t word = 0;
#pragma unroll
              for (int j = 0; j < 4; ++j) word |= f32_to_e4m3(h[tt][j] / scale) << (8 * j);
              const size_t r = (size_t)(c.it.rows0 + col);
              *reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(c.it.out) + r * Nout + cfirst) = word;
              if (ft == 0 && lane < 16) c.it.out_scale[r * (Nout / 128) + c.it.col0 / 128] = scale;
            }
          }
        }
      } else if (kp == 0) {
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
          const int col = tt * 16 + r16;
          if (col < c.it.nrows) {
            const size_t r = (size_t)(c.it.rows0 + col);
            if constexpr (OUT == MOE_F32) {
              *reinterpret_cast<f32x4_t*>(static_cast<float*>(c.it.out) + r * Nout + cfirst) =
                  f32x4_t{h[tt][0], h[tt][1], h[tt][2], h[tt][3]};
            } else {
              const uint32_t lo = f32_to_bf16_bits(h[tt][0]) | (f32_to_bf16_bits(h[tt][1]) << 16);
              const uint32_t hi = f32_to_bf16_bits(h[tt][2]) | (f32_to_bf16_bits(h[tt][3]) << 16);
              *reinterpret_cast<uint2*>(static_cast<uint16_t*>(c.it.out) + r * Nout + cfirst) =
                  make_uint2(lo, hi);
            }
          }
        }
      }
    } else if (kp == 0) {
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        const int col = tt * 16 + r16;
        if (col < c.it.nrows) {
          const size_t r = (size_t)(c.it.rows0 + col);
#pragma unroll
          for (int m = 0; m < NMAT; ++m)
            *reinterpret_cast<f32x4_t*>(static_cast<float*>(c.it.out) + r * Nout + cfirst + 16 * m) = acc[m][tt];
        }
      }
    }
    if constexpr (KS > 1 || OUT == MOE_FP8_E4M3) __syncthreads();  // LDS is reused by the next finish
  };

  // Main loop, three stages per iteration.  The stages are straight-line
  // code (loads two stages ahead, MFMAs on the current one); an item that
  // ends inside the iteration parks its accumulator and is finished at the
  // bottom of the iteration, so no store or barrier sits between a load and its use.
  // Past the end the cursors stay on their last stage: the extra loads and
  // MFMAs are harmless and nothing is parked for them.
  Cursor ic, cc;
  walk.start(ic, bid);
  walk.start(cc, bid);
  bool idone = false, cdone = false;
  St ring[3];
  load(ring[0], ic);
  walk.advance(ic, idone);
  load(ring[1], ic);
  walk.advance(ic, idone);
  zero_acc();
  if constexpr (!PARK) {
    // no parked accumulators: an item is finished right after its last
    // stage (its loads for the next two stages are already in flight).
    // Stage n sits in ring[n % 3] and, shared, in LDS slot n % 3; slot
    // (n + 1) % 3 is rewritten at stage n, after the barrier of stage n - 1
    // that every wave passes only once done with stage n - 2.
    if constexpr (SHARE) {
      put(ring[0], 0);
      lds_barrier();
    }
    while (!cdone) {
#pragma unroll
      for (int r = 0; r < 3; ++r) {
        const bool live = !cdone;
        load(ring[(r + 2) % 3], ic);
        walk.advance(ic, idone);
        if constexpr (SHARE) {
          put(ring[(r + 1) % 3], (r + 1) % 3);
          lds_barrier();
        }
        compute(ring[r], cc, r);
        if (live && cc.step == cc.it.s_end - 1) {
          finish(acc, cc);
          zero_acc();
        }
        if (live) walk.advance(cc, cdone);
      }
    }
    return;
  }
  if constexpr (SHARE) {  // slots as in the walk above
    put(ring[0], 0);
    lds_barrier();
  }
  while (!cdone) {
    bool parked[3];
    Cursor pc[3];
    f32x4_t pacc[3][NMAT][TT];
#pragma unroll
    for (int r = 0; r < 3; ++r) {
      const bool live = !cdone;
      load(ring[(r + 2) % 3], ic);
      walk.advance(ic, idone);
      if constexpr (SHARE) {
        put(ring[(r + 1) % 3], (r + 1) % 3);
        lds_barrier();
      }
      compute(ring[r], cc, r);
      parked[r] = live && cc.step == cc.it.s_end - 1;
      if (parked[r]) {
        pc[r] = cc;
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
          for (int tt = 0; tt < TT; ++tt) pacc[r][m][tt] = acc[m][tt];
        zero_acc();
      }
      if (live) walk.advance(cc, cdone);
    }
#pragma unroll
    for (int r = 0; r < 3; ++r)
      if (parked[r]) finish(pacc[r], pc[r]);
  }
}

template <int DT, int FW, int KS, int TT, bool GATED, int OUT, int NM, bool PARK = true, bool SHARE = false>
__global__ __launch_bounds__(64 * FW * KS) void ffn_kernel(FfnParams p) {
  ffn_body<DT, FW, KS, TT, GATED, OUT, NM, PARK, SHARE>(p, blockIdx.x, gridDim.x);
}

// Residency of the bf16 and f32 walks: one workgroup per CU.  Each wave
// keeps three K-steps of loads in flight, so one workgroup of 2-4 waves
// already draws a CU's share of HBM bandwidth; more resident workgroups only
// add L2 and address-unit contention (measured: 2.5-4% faster on 128-expert
// decode and up to 4% on 256-expert; a cap of two gained nothing).  The cap
// is an unused dynamic LDS reservation sized so a second workgroup cannot
// fit.  The E4M3 walks stay at full occupancy: their dequantising down pass
// measured no better under the cap.
#ifndef MOE_FFN_RESIDENT
#define MOE_FFN_RESIDENT 1
#endif
static constexpr int kResidentCap = MOE_FFN_RESIDENT;

template <int DT, int FW, int KS, int TT, bool GATED, int OUT, int NM = 2, bool PARK = true, bool SHARE = false>
static hipError_t launch_one(const FfnParams& p, long long max_items, hipStream_t stream) {
  auto kern = ffn_kernel<DT, FW, KS, TT, GATED, OUT, NM, PARK, SHARE>;
  // constant per kernel and device model: computed once, on the first call
  // (thread-safe initialisation of a const local static)
  static const Residency occ = [&] {
    Residency o{};
    int dev = 0, n = 0, c = 0, lds = 0;
    if (hipGetDevice(&dev) != hipSuccess) return o;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) c = 256;
    if (DT != MOE_FP8_E4M3 && kResidentCap > 0 &&
        hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) == hipSuccess &&
        lds > 0) {
      const size_t r = (size_t)lds / (kResidentCap + 1) + 1;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, 64 * FW * KS, r) == hipSuccess && n >= 1)
        o.reserve = r;
    }
    if (o.reserve == 0 && hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, 64 * FW * KS, 0) != hipSuccess)
      n = 1;
    o.cus = c;
    o.per_cu = n > 0 ? n : 1;
    o.ok = true;
    return o;
  }();
  if (!occ.ok) return hipErrorInvalidDevice;
  const long long cap = (long long)occ.per_cu * occ.cus;
  const int grid = (int)(max_items < cap ? max_items : cap);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * FW * KS), occ.reserve, stream, p);
  return hipGetLastError();
}

// Launch shape of a pass: FW column tiles x KS reduction splits per
// workgroup, 16-row token tiles (one per item).  KS must not exceed the K-steps of any
// item (every wave needs at least one step per item).  The MOE_FFN_* macros
// pin a shape for launch-shape sweeps.
struct Plan {
  int fw, ks;
};

static Plan plan_of(const FfnParams& p, int step, bool gated, int wdtype) {
  int steps = p.K_r / step;
  if (p.n_shared && p.K_s / step < steps) steps = p.K_s / step;
  // Long reductions are split over 4 waves (keeps enough waves busy when few
  // experts have rows); shorter ones keep more steps per wave instead.
  Plan pl{1, 4};
  if (steps < 32) pl = steps >= 8 ? Plan{2, 2} : Plan{gated ? 4 : 2, 1};
  if (steps < pl.ks) pl = Plan{gated ? 4 : 2, 1};
  if (gated && wdtype == MOE_FP8_E4M3) pl = Plan{8, 1};
#ifdef MOE_FFN_FW
  if (!(gated && wdtype == MOE_FP8_E4M3)) pl.fw = MOE_FFN_FW;
#endif
#ifdef MOE_FFN_KS
  if (!(gated && wdtype == MOE_FP8_E4M3)) pl.ks = MOE_FFN_KS < steps ? MOE_FFN_KS : steps;
#endif
  return pl;
}

template <int DT, bool GATED, int OUT, int TT = 1, bool PARK = true, bool SHARE = false>
static hipError_t launch_plan(const FfnParams& p, const Plan& pl, long long items, hipStream_t stream) {
#define MOE_FFN_CASE(FW, KS)           \
  if (pl.fw == FW && pl.ks == KS)      \
    return launch_one<DT, FW, KS, TT, GATED, OUT, 2, PARK, SHARE>(p, items, stream);
  MOE_FFN_CASE(1, 4)
  MOE_FFN_CASE(1, 2)
  MOE_FFN_CASE(1, 1)
  MOE_FFN_CASE(8, 1)
  MOE_FFN_CASE(4, 1)
  MOE_FFN_CASE(2, 2)
  MOE_FFN_CASE(2, 1)
#undef MOE_FFN_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_ffn(const FfnParams& p, int wdtype, bool gated, long long routed_rows, int max_groups,
                      hipStream_t stream) {
  const int step = wdtype == MOE_F32 ? 64 : wdtype == MOE_BF16 ? 128 : 256;
  if (p.K_r / step < 1 || (p.n_shared && p.K_s / step < 1)) return hipErrorInvalidValue;
  Plan pl = plan_of(p, step, gated, wdtype);
  // E4M3 batches with many rows per expert (T k >= 12 E) use 32-row chunks:
  // each weight tile is then streamed once per 32 rows instead of once per 16
  // (measured at 512 tokens x 8 of 256 experts: gate/up 2036 -> 1792 us; at
  // 128 tokens the 16-row chunks are faster).  The wider activation tiles
  // leave no registers for parked accumulators, so those walks finish each
  // item in line.
  const bool wide = wdtype == MOE_FP8_E4M3 && routed_rows >= 12LL * max_groups;
#ifndef MOE_FFN_FW
  // Once experts hold a few rows each, the E4M3 down pass does better with
  // more column waves sharing each activation tile and no K-split.  Measured
  // at 256 experts x 8 slots, down pass with (2, 2) / (4, 1) / (8, 1): 512
  // tokens 782 / 710 / 686 us; 128 tokens 506 / 489 / 494 us; 32 tokens (one
  // row per expert) 322 / 326 / 335 us.
  if (!gated && wdtype == MOE_FP8_E4M3 && routed_rows >= 2LL * max_groups) {
    for (const Plan w : {wide ? Plan{8, 1} : Plan{4, 1}, Plan{4, 1}})
      if (p.tiles_r % (2 * w.fw) == 0 && p.tiles_s % (2 * w.fw) == 0) {
        pl = w;
        break;
      }
  }
  // A bf16 gated pass of 16-31 steps with under two rows per touched expert
  // and at least 32 of them: one column wave per item and a 4-way K-split.
  // Measured at 128 experts x 8 slots, d_model = 2048, (2, 2) against (1, 4),
  // two runs each: 8 tokens 62.1, 62.3 / 58.7, 59.1 us.  It loses at 1 token
  // (8 experts: 19.3, 19.5 / 20.8, 20.1 us) and from 32 tokens on (126.5,
  // 126.3 / 131.4, 131.5 us; 128 tokens 141.9, 142.2 / 153.8, 153.9 us).
  // Not with a shared expert, whose items moe_layer may run in the router's
  // launch with the shape of plan_of.
  if (gated && wdtype == MOE_BF16 && !p.n_shared && max_groups >= 32 && routed_rows < 2LL * max_groups &&
      p.K_r / step >= 16 && p.K_r / step < 32)
    pl = Plan{1, 4};
  // A bf16 plain pass with short items (under 16 steps) and eight or more
  // rows per touched expert: four column waves sharing each activation tile.
  // Measured at 128 experts x 8 slots, d_ff = 768 (6 steps), down pass with
  // (2, 1) private / (4, 1) shared tiles, two runs each: 128 tokens
  // 80.7, 81.3 / 78.7, 78.5 us; 256 tokens 108.5, 109.3 / 99.5, 100.0 us.
  // With fewer rows per expert the tiles are mostly padding and sharing them
  // does not pay (32 tokens: 67.7 against 71.6 us).
  const bool dense_plain = !gated && wdtype == MOE_BF16 && routed_rows >= 8LL * max_groups;
  if (dense_plain) {
    int st = p.K_r / step;
    if (p.n_shared && p.K_s / step < st) st = p.K_s / step;
    if (st < 16 && p.tiles_r % 8 == 0 && p.tiles_s % 8 == 0) pl = Plan{4, 1};
  }
#endif
  // a work item covers FW waves' columns; a plain-pass wave covers two tiles
  const int per_item = pl.fw * (gated ? 1 : 2);
  FfnParams q = p;
  q.tiles_r = p.tiles_r / per_item;
  q.tiles_s = p.tiles_s / per_item;
  if (q.tiles_r * per_item != p.tiles_r || q.tiles_s * per_item != p.tiles_s) return hipErrorInvalidValue;
  const int CH = wide ? 32 : 16;
  // CH-row chunks over all groups: full chunks plus at most one partial
  // chunk per group (bounds the items, which sizes the grid)
  const long long chunks_r = routed_rows / CH + max_groups;
  const long long chunks_s = q.n_shared ? (q.T + CH - 1) / CH : 0;
  const long long items = chunks_r * q.tiles_r + chunks_s * q.tiles_s;
  if (items <= 0) return hipSuccess;
  if (wdtype == MOE_F32) {
    if (gated) return launch_plan<MOE_F32, true, MOE_F32>(q, pl, items, stream);
    return launch_plan<MOE_F32, false, MOE_F32>(q, pl, items, stream);
  }
  // every wave of a workgroup walks the same number of steps per item
  const bool even = (q.K_r / step) % pl.ks == 0 && (!q.n_shared || (q.K_s / step) % pl.ks == 0);
  if (wdtype == MOE_BF16) {
    // bf16 tiles are shared between column waves of items with 16 or more
    // steps: measured at 128 tokens, 128 experts: gate/up (16 steps) 143.0 ->
    // 141.5 us, but the 6-step down pass with (2, 1) 80.4 -> 84.2 us; 256
    // experts: down (16 steps) 941 -> 916 us.  Short dense plain passes share
    // under the (4, 1) shape chosen above.
    int steps = q.K_r / step;
    if (q.n_shared && q.K_s / step < steps) steps = q.K_s / step;
#ifndef MOE_FFN_FW
    const bool dense4 = dense_plain && pl.fw == 4 && pl.ks == 1;
#else
    const bool dense4 = false;
#endif
    if ((pl.fw >= 2 && steps >= 16 && even) || dense4) {
      if (gated) return launch_plan<MOE_BF16, true, MOE_BF16, 1, true, true>(q, pl, items, stream);
      return launch_plan<MOE_BF16, false, MOE_F32, 1, true, true>(q, pl, items, stream);
    }
    if (gated) return launch_plan<MOE_BF16, true, MOE_BF16>(q, pl, items, stream);
    return launch_plan<MOE_BF16, false, MOE_F32>(q, pl, items, stream);
  }
  if (wide) {
    // The waves of a workgroup share each step's 32-row activation tile
    // through LDS (measured upper bound, with the activation loads removed
    // altogether at 512 tokens: gate/up 1803 -> 1229 us, down 923 -> 717 us).
    // Sharing needs every wave to walk the same number of steps per item, so
    // the K-split must divide every item's steps.
    if (gated) return launch_one<MOE_FP8_E4M3, 8, 1, 2, true, MOE_FP8_E4M3, 2, false, true>(q, items, stream);
    if (even) return launch_plan<MOE_FP8_E4M3, false, MOE_F32, 2, false, true>(q, pl, items, stream);
    return launch_plan<MOE_FP8_E4M3, false, MOE_F32, 2, false>(q, pl, items, stream);
  }
  // 16-row chunks share their tiles too (measured upper bound at 128 tokens:
  // gate/up 1005 -> 932 us, down 534 -> 488 us)
  if (gated) return launch_one<MOE_FP8_E4M3, 8, 1, 1, true, MOE_FP8_E4M3, 2, true, true>(q, items, stream);
  if (even) return launch_plan<MOE_FP8_E4M3, false, MOE_F32, 1, true, true>(q, pl, items, stream);
  return launch_plan<MOE_FP8_E4M3, false, MOE_F32>(q, pl, items, stream);
}

// The router GEMM at decode: its weight is small (E x d), so an item is one
// 16-column tile (NM = 1) and the reduction is split eight ways inside the
// workgroup, which spreads it over E / 16 workgroups of eight waves.
template <int DT>
static hipError_t launch_router_dt(const FfnParams& q, long long items, int steps, hipStream_t stream) {
  if (steps >= 8) return launch_one<DT, 1, 8, 1, false, MOE_F32, 1>(q, items, stream);
  if (steps >= 4) return launch_one<DT, 1, 4, 1, false, MOE_F32, 1>(q, items, stream);
  return launch_one<DT, 1, 1, 1, false, MOE_F32, 1>(q, items, stream);
}

hipError_t launch_router_gemm(const FfnParams& p, int dtype, hipStream_t stream) {
  const int step = dtype == MOE_F32 ? 64 : 128;
  if (p.E != 0 || !p.masked || p.n_shared != 1 || p.Nout_s % 16 || p.K_s % step) return hipErrorInvalidValue;
  FfnParams q = p;
  q.tiles_r = 0;
  q.tiles_s = p.Nout_s / 16;
  const long long items = (long long)(p.T + 15) / 16 * q.tiles_s;
  const int steps = p.K_s / step;
  if (dtype == MOE_F32) return launch_router_dt<MOE_F32>(q, items, steps, stream);
  if (dtype == MOE_BF16) return launch_router_dt<MOE_BF16>(q, items, steps, stream);
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// The router next to the shared expert's gate/up pass, in one launch
// ("Hot-Expert Skew" section, shared experts; the shared expert needs no
// routing).  The first nroute workgroups route four tokens each (one, and
// write it, in the masked layout); the others run the persistent gate/up
// walk over the shared expert's items only (sp has no routed groups),
// streaming its weights while HBM would otherwise idle behind the router.  bf16 only: on the E4M3 path the shared expert reads the
// tokens the dispatch quantises.
// ---------------------------------------------------------------------------

template <int KPL, int FW, int KS>
__global__ __launch_bounds__(64 * FW * KS) void route_shared_kernel(RouteParams rp, FfnParams sp, int nroute) {
  extern __shared__ float smem[];
  static_assert(FW * KS == 4, "the routing workgroups hold four waves");
  if ((int)blockIdx.x < nroute) {
    if (rp.fuse) route_dispatch_block<KPL>(rp, blockIdx.x, smem);  // one token, masked-layout write
    else route_body<KPL, 4>(rp, blockIdx.x, smem);                 // four tokens
  } else
    ffn_body<MOE_BF16, FW, KS, 1, true, MOE_BF16, 2>(sp, blockIdx.x - nroute, gridDim.x - nroute);
}

template <int KPL, int FW, int KS>
static hipError_t launch_rs(const RouteParams& rp, const FfnParams& q, long long items, hipStream_t stream) {
  auto kern = route_shared_kernel<KPL, FW, KS>;
  constexpr int NT = 64 * FW * KS;
  const size_t lds = (size_t)(FW * KS) * route_lds_floats(rp.E) * sizeof(float);
  // workgroups per CU for the largest routing LDS (E = 1024), constant per
  // kernel and device model: computed once (thread-safe static initialisation)
  static const Residency occ = [&] {
    Residency o{};
    int dev = 0, n = 0, c = 0;
    if (hipGetDevice(&dev) != hipSuccess) return o;
    const size_t lds_max = (size_t)(FW * KS) * route_lds_floats(1024) * sizeof(float);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, NT, lds_max) != hipSuccess || n < 1) n = 1;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) c = 256;
    o.per_cu = n;
    o.cus = c;
    o.ok = true;
    return o;
  }();
  if (!occ.ok) return hipErrorInvalidDevice;
  const long long cap = (long long)occ.per_cu * occ.cus;
  const int nroute = rp.fuse ? rp.T : (rp.T + FW * KS - 1) / (FW * KS);
  const int nshared = (int)(items < cap ? items : cap);
  hipLaunchKernelGGL(kern, dim3(nroute + nshared), dim3(NT), lds, stream, rp, q, nroute);
  return hipGetLastError();
}

bool route_shared_supported(const FfnParams& sp, int wdtype) {
  if (wdtype != MOE_BF16 || !sp.n_shared) return false;
  const Plan pl = plan_of(sp, 128, true, wdtype);
  return (pl.fw == 1 && pl.ks == 4) || (pl.fw == 2 && pl.ks == 2);
}

hipError_t launch_route_shared(const RouteParams& rp, const FfnParams& sp, int wdtype, hipStream_t stream) {
  if (!route_shared_supported(sp, wdtype)) return hipErrorInvalidValue;
  const Plan pl = plan_of(sp, 128, true, wdtype);
  FfnParams q = sp;
  q.E = 0;  // no routed groups: the walk covers the shared expert only
  q.tiles_r = sp.tiles_r / pl.fw;
  q.tiles_s = sp.tiles_s / pl.fw;
  if (q.tiles_s * pl.fw != sp.tiles_s) return hipErrorInvalidValue;
  const long long items = (long long)(q.T + 15) / 16 * q.tiles_s;
  const int kpl = (rp.E + 63) / 64;
#define MOE_RS_CASE(K)                                                          \
  if (kpl <= K) {                                                               \
    if (pl.fw == 1) return launch_rs<K, 1, 4>(rp, q, items, stream);            \
    return launch_rs<K, 2, 2>(rp, q, items, stream);                            \
  }
  MOE_RS_CASE(1)
  MOE_RS_CASE(2)
  MOE_RS_CASE(4)
  MOE_RS_CASE(8)
  MOE_RS_CASE(16)
#undef MOE_RS_CASE
  return hipErrorInvalidValue;
}

}  // namespace moe
