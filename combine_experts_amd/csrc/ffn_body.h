// Weight-streaming grouped GEMM walk over the dispatch layout (device code),
// shared by the decode GEMM kernels, the router-with-shared-expert launch
// and the fused decode layer.  The design notes are at the top of ffn.hip.
#pragma once

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
  float xsp[2];        // shared tile: one row's two activation scales, on their way to LDS
  float sw[NMAT][2];   // E4M3 weight block scales of the step
};

// Everything about one item that the loads and the epilogue need; all fields
// are uniform across the wave.
struct Item {
  int valid;
  int rows0, nrows, K, Nout, col0, s_begin, s_end, rot;
  const uint8_t* w;
  const uint8_t* act;
  const int* gather;  // activation row r is act row gather[r] (routed groups of a gathering walk), or r
  const float* act_scale;
  const float* w_scale;
  void* out;
  float* out_scale;
};

struct Cursor {
  Item it;
  int item, step;
};

template <int DT, int FW, int KS, int TT, int WC, bool GATHER = false>
struct Walker {
  static constexpr int ES = Elem<DT>::kBytes;
  static constexpr int STEP = Elem<DT>::kStep;
  const FfnParams& p;
  const int* s_off;
  const int* s_act;
  const int* s_pre;  // items before active group a; s_pre[n_active] = routed items
  int n_active, n_routed_items, n_items, ft, kp, nblk;
  bool single;  // every active group is one chunk: group a owns items [a tiles_r, (a+1) tiles_r)
  const int* gather;  // see Item::gather; nullptr: rows are read in place

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
      nrows = p.masked ? min(uni(s_off[g]), p.T) : uni(s_off[g + 1]) - rows0;
      K = p.K_r;
      it.Nout = p.Nout_r;
      it.w = p.w + (size_t)g * p.NW_r * K * ES;
      it.act = p.act;
      it.act_scale = p.act_scale;
      it.w_scale = p.w_scale ? p.w_scale + (size_t)g * (p.NW_r / 128) * (K / 128) : nullptr;
      it.out = p.out;
      it.out_scale = p.out_scale;
      if constexpr (GATHER) it.gather = gather;
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
      if constexpr (GATHER) it.gather = nullptr;
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
// in the same order.  E4M3 walks share the step's activation scales the same
// way: the first TT*16 lanes of the K-split part load one row's pair each,
// instead of every wave loading all rows' pairs (a 4- or 8-byte load per
// row, each a cache-line request of its own).
//
// GATHER (the fused layer): the compact-layout offsets [E+1] come from
// off_src instead of p.expert_offset (the caller routed in LDS), and routed
// activation row r is read from row gather[r] of p.act (the tokens
// themselves instead of dispatched rows).  Without it the arguments are
// unused and the walk is the plain one.
template <int DT, int FW, int KS, int TT, bool GATED, int OUT, int NM, bool PARK = true, bool SHARE = false,
          bool GATHER = false>
__device__ __forceinline__ void ffn_body(const FfnParams& p, int bid, int nblk, const int* off_src = nullptr,
                                         const int* gather = nullptr) {
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
  using W = Walker<DT, FW, KS, TT, WC, GATHER>;
  using St = Stage<DT, NMAT, TT, NX, XP>;
  __shared__ float red[RED];
  // three stage slots per K-split part, rows XOR-swizzled in 16-byte units
  __shared__ __attribute__((aligned(16))) uint8_t xs[SHARE ? 3 * KS * XT : 16];
  constexpr bool SSC = SHARE && FP8;  // shared activation scales
  __shared__ float2 xsc[SSC ? 3 * KS * TT * 16 : 1];
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
  for (int e = tid; e <= E; e += NT) {
    if constexpr (GATHER) s_off[e] = off_src[e];
    else s_off[e] = p.masked ? (e < E ? p.expert_offset[e] : 0) : p.expert_offset[e];
  }
  __syncthreads();
  constexpr int CH = TT * 16;  // rows per chunk
  {
    const int per = (E + NT - 1) / NT;
    const int e0 = tid * per;
    int cnt = 0, items = 0;
    for (int i = 0; i < per; ++i) {
      const int e = e0 + i;
      if (e < E) {
        const int n = p.masked ? min(s_off[e], p.T) : s_off[e + 1] - s_off[e];
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
        const int n = p.masked ? min(s_off[e], p.T) : s_off[e + 1] - s_off[e];
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
               routed_items == n_active * p.tiles_r, gather};
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
        int arow = c.it.rows0 + row;
        if constexpr (GATHER) arow = c.it.gather ? c.it.gather[arow] : arow;
        const uint8_t* src = c.it.act + (size_t)arow * rowbytes + (size_t)ps * 256 + (i % PPR) * PB;
        if constexpr (PB == 16) {
          s.xp[q] = *reinterpret_cast<const i32x4_t*>(src);
        } else {
          const uint2 v = *reinterpret_cast<const uint2*>(src);
          s.xp[q] = i32x4_t{(int)v.x, (int)v.y, 0, 0};
        }
      }
      if constexpr (SSC) {
        const int i = ft * 64 + lane;  // row of the tile whose scales this lane loads
        if (i < TT * 16) {
          int arow = c.it.rows0 + (i < c.it.nrows ? i : 0);  // rows past the group's end: never stored
          if constexpr (GATHER) arow = c.it.gather ? c.it.gather[arow] : arow;
          const float* sp = c.it.act_scale + (size_t)arow * (c.it.K / 128) + 2 * ps;
          s.xsp[0] = sp[0];
          s.xsp[1] = sp[1];
        }
      }
    }
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
      const int ps = walk.phys(c);
      const int row = (GATED ? (m == 0 ? 0 : c.it.Nout) : 16 * m) + c.it.col0 + r16;
      load_step(s.w[m], c.it.w + (size_t)row * rowbytes + (size_t)ps * 256, lane);
      if constexpr (FP8) {
        // the block scales are the same for the whole wave and never written
        // during the launch: scalar loads (constant address space), so the
        // vector-memory path carries only the tiles
        const int wsrow = ((GATED ? (m == 0 ? 0 : c.it.Nout) : 16 * m) + c.it.col0) / 128;
        const float* wsp = c.it.w_scale + (size_t)wsrow * (c.it.K / 128) + 2 * ps;
        typedef const __attribute__((address_space(4))) float cfloat;
        const cfloat* q = (const cfloat*)(uintptr_t)wsp;
        s.sw[m][0] = q[0];
        s.sw[m][1] = q[1];
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
        size_t arow = row;
        if constexpr (GATHER) arow = c.it.gather ? (size_t)c.it.gather[row] : row;
        if constexpr (!SHARE) load_step(s.x[xi][tt], c.it.act + arow * rowbytes + (size_t)ps * 256, lane);
        if constexpr (FP8 && !SSC) {
          const float* sp = c.it.act_scale + arow * (c.it.K / 128) + 2 * ps;
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
      if constexpr (SSC) {
        const int i = ft * 64 + lane;
        if (i < TT * 16) xsc[(slot * KS + kp) * TT * 16 + i] = make_float2(s.xsp[0], s.xsp[1]);
      }
    }
  };
  // activation scales of token tile tt's row (lane % 16) at a stage
  auto xscale = [&](const St& s, int slot, int tt) {
    if constexpr (SSC) {
      return xsc[(slot * KS + kp) * TT * 16 + tt * 16 + r16];
    } else {
      return make_float2(s.sx[0][tt][0], s.sx[0][tt][1]);
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
    if constexpr (FP8 && SHARE && TT > 2) {
      // 64-row chunks: one token block's operand at a time, read from the
      // LDS slot just before its MFMAs (holding all four would not fit)
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        if (tt * 16 < left) {
          const Step xv = xstep(s, slot, tt);
#pragma unroll
          for (int m = 0; m < NMAT; ++m) {
            const f32x4_t p0 = mma_fp8_block(s.w[m], xv, 0);
            const f32x4_t p1 = mma_fp8_block(s.w[m], xv, 1);
            const float2 sx = xscale(s, slot, tt);
            const float c0 = s.sw[m][0] * sx.x, c1 = s.sw[m][1] * sx.y;
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[m][tt][j] += p0[j] * c0 + p1[j] * c1;
          }
        }
      }
      return;
    }
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
            const float2 sx = xscale(s, slot, tt);
            const float c0 = sw0 * sx.x, c1 = sw1 * sx.y;
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

}  // namespace moe
