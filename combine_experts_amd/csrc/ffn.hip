// Grouped expert GEMMs over the dispatch buffer (read in place) and the shared
// expert.  "7.13 Serving Mixture-of-Experts", section "Expert Parallelism
// Mechanics", step 3: one grouped GEMM runs all local experts' matmuls in a
// single launch; section "Prefill vs. Decode": at decode each expert sees a
// handful of rows, so the pass is bound by streaming the touched experts'
// weights.
//
// Design (gfx950): the weights are the MFMA A operand and go straight from
// HBM into registers, 256 bytes of each of 16 rows per step and lane group;
// the activation rows are the B operand (16 tokens per tile).  A workgroup
// owns one (group, tile) item; its KS waves split the reduction dimension and
// are summed through LDS in a fixed order, so results do not depend on timing.
// Experts with no rows own no items and their weights are never read.
#include "moe_kernels.h"

namespace moe {

// Find this block's item: the rank-a non-empty expert, and the number of
// non-empty experts.  Wave 0 scans expert_offset (E <= 1024, 16 per lane).
__device__ __forceinline__ void find_group(const int* off, int E, int a, int* out_group, int* out_nactive) {
  const int lane = threadIdx.x & 63;
  int cnt = 0;
  const int e0 = lane * 16;
  int prev = e0 < E ? off[e0] : 0;
#pragma unroll 4
  for (int i = 0; i < 16; ++i) {
    const int e = e0 + i;
    if (e < E) {
      const int nxt = off[e + 1];
      cnt += nxt > prev ? 1 : 0;
      prev = nxt;
    }
  }
  int inc = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(inc, o);
    if (lane >= o) inc += y;
  }
  const int total = __shfl(inc, 63);
  const int before = inc - cnt;
  if (lane == 0) *out_nactive = total;
  if (a >= before && a < inc) {
    int seen = before;
    prev = off[e0];
    for (int i = 0; i < 16; ++i) {
      const int e = e0 + i;
      const int nxt = off[e + 1];
      if (nxt > prev) {
        if (seen == a) { *out_group = e; break; }
        ++seen;
      }
      prev = nxt;
    }
  }
}

template <int DT, int NMAT, int TT>
struct Regs {
  Step w[NMAT];
  Step x[TT];
  float sx[TT][2];  // E4M3 activation scales of the step's two 128-blocks
};

template <int DT, int FW, int KS, int TT, bool GATED, int OUT>
__global__ __launch_bounds__(64 * FW * KS) void ffn_kernel(FfnParams p) {
  constexpr int NMAT = GATED ? 2 : 1;
  constexpr int ES = Elem<DT>::kBytes;
  constexpr int STEP = Elem<DT>::kStep;
  constexpr bool FP8 = DT == MOE_FP8_E4M3;
  constexpr int RED = (KS > 1 ? (KS - 1) : 1) * FW * NMAT * TT * 4 * 64;
  __shared__ float red[RED];
  __shared__ float amax_s[FW][TT * 16];
  __shared__ int s_group, s_nactive;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wid = tid >> 6;
  const int ft = wid % FW, kp = wid / FW;

  // ---- resolve the item
  if (wid == 0) {
    if (lane == 0) s_group = -1;
    // lane 0's write must land before find_group's writes
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    int a = (int)(blockIdx.x / p.tiles_r);
    find_group(p.expert_offset, p.E, a, &s_group, &s_nactive);
  }
  __syncthreads();
  const int n_active = s_nactive;
  int item = blockIdx.x;
  bool shared;
  int g, tile;
  if (item < n_active * p.tiles_r) {
    shared = false;
    g = s_group;
    tile = item % p.tiles_r;
  } else {
    item -= n_active * p.tiles_r;
    if (item >= p.n_shared * p.tiles_s) return;  // uniform per block
    shared = true;
    g = 0;
    tile = item;
  }

  int rows0, nrows, K, Nout;
  const uint8_t *act, *wmat;
  const float *act_scale = nullptr, *w_scale = nullptr;
  void* out;
  float* out_scale;
  size_t wrows;
  if (!shared) {
    rows0 = p.expert_offset[g];
    nrows = p.expert_offset[g + 1] - rows0;
    K = p.K_r;
    Nout = p.Nout_r;
    wrows = (size_t)p.NW_r;
    act = p.act;
    wmat = p.w + (size_t)g * wrows * K * ES;
    if (FP8) {
      act_scale = p.act_scale;
      w_scale = p.w_scale + (size_t)g * (wrows / 128) * (K / 128);
    }
    out = p.out;
    out_scale = p.out_scale;
  } else {
    rows0 = 0;
    nrows = p.T;
    K = p.K_s;
    Nout = p.Nout_s;
    wrows = (size_t)p.NW_s;
    act = p.s_act;
    wmat = p.s_w;
    if (FP8) {
      act_scale = p.s_act_scale;
      w_scale = p.s_w_scale;
    }
    out = p.s_out;
    out_scale = p.s_out_scale;
  }

  const int col0 = tile * 16 * FW + ft * 16;  // first output column of this wave
  const size_t rowbytes = (size_t)K * ES;
  const uint8_t* wrow[NMAT];
  wrow[0] = wmat + (size_t)(col0 + (lane & 15)) * rowbytes;
  if (GATED) wrow[NMAT - 1] = wmat + (size_t)(Nout + col0 + (lane & 15)) * rowbytes;
  const int ksb = K / 128;  // 128-column scale blocks per row
  int wsrow[NMAT];          // first scale row of each matrix tile (E4M3)
  wsrow[0] = col0 / 128;
  if (GATED) wsrow[NMAT - 1] = (Nout + col0) / 128;

  const int steps = K / STEP;
  const int s_begin = kp * steps / KS, s_end = (kp + 1) * steps / KS;

  for (int chunk = 0; chunk < nrows; chunk += TT * 16) {
    // activation rows of this lane's token column in each tile
    const uint8_t* xrow[TT];
    bool xval[TT];
    int ntile = 0;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const int c = chunk + tt * 16 + (lane & 15);
      xval[tt] = c < nrows;
      xrow[tt] = act + (size_t)(rows0 + (xval[tt] ? c : 0)) * rowbytes;
      if (chunk + tt * 16 < nrows) ntile = tt + 1;
    }

    f32x4_t acc[NMAT][TT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) acc[m][tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    auto load = [&](Regs<DT, NMAT, TT>& r, int s) {
      const size_t kb = (size_t)s * 256;
#pragma unroll
      for (int m = 0; m < NMAT; ++m) load_step(r.w[m], wrow[m] + kb, lane);
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        if (tt < ntile) {
          if (xval[tt]) {
            load_step(r.x[tt], xrow[tt] + kb, lane);
            if (FP8) {
              const float* sp = act_scale + (size_t)(rows0 + chunk + tt * 16 + (lane & 15)) * ksb + 2 * s;
              r.sx[tt][0] = sp[0];
              r.sx[tt][1] = sp[1];
            }
          } else {
            zero_step(r.x[tt]);
            if (FP8) { r.sx[tt][0] = 0.f; r.sx[tt][1] = 0.f; }
          }
        }
      }
    };
    auto compute = [&](const Regs<DT, NMAT, TT>& r, int s) {
      if constexpr (FP8) {
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
          const float* wsp = w_scale + (size_t)wsrow[m] * ksb + 2 * s;
          const float sw0 = wsp[0], sw1 = wsp[1];
#pragma unroll
          for (int tt = 0; tt < TT; ++tt) {
            if (tt < ntile) {
              const f32x4_t p0 = mma_fp8_block(r.w[m], r.x[tt], 0);
              const f32x4_t p1 = mma_fp8_block(r.w[m], r.x[tt], 1);
              const float c0 = sw0 * r.sx[tt][0], c1 = sw1 * r.sx[tt][1];
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
            if (tt < ntile) Mma<DT>::run(acc[m][tt], r.w[m], r.x[tt]);
      }
    };

    // software pipeline: the next step's loads are in flight during this step's MFMAs
    if (s_begin < s_end) {
      Regs<DT, NMAT, TT> ra, rb;
      int s = s_begin;
      load(ra, s);
      while (true) {
        if (s + 1 < s_end) load(rb, s + 1);
        compute(ra, s);
        if (++s >= s_end) break;
        if (s + 1 < s_end) load(ra, s + 1);
        compute(rb, s);
        if (++s >= s_end) break;
      }
    }

    // ---- reduce the KS partial sums (fixed order kp = 1, 2, ...)
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

    // ---- epilogue: lane holds output columns col0 + 4 (lane/16) + j of token
    // column chunk + tt*16 + lane%16
    const int cfirst = col0 + 4 * (lane >> 4);
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
            const int c = chunk + tt * 16 + (lane & 15);
            if (c < nrows) {
              float a = 0.f;
#pragma unroll
              for (int f = 0; f < FW; ++f) a = fmaxf(a, amax_s[f][tt * 16 + (lane & 15)]);
              const float scale = a > 0.f ? a / 448.0f : 1.0f;
              uint32_t word = 0;
#pragma unroll
              for (int j = 0; j < 4; ++j) word |= f32_to_e4m3(h[tt][j] / scale) << (8 * j);
              const size_t r = (size_t)(rows0 + c);
              *reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(out) + r * Nout + cfirst) = word;
              if (ft == 0 && lane < 16) out_scale[r * (Nout / 128) + col0 / 128] = scale;
            }
          }
        }
      } else if (kp == 0) {
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
          const int c = chunk + tt * 16 + (lane & 15);
          if (c < nrows) {
            const size_t r = (size_t)(rows0 + c);
            if constexpr (OUT == MOE_F32) {
              *reinterpret_cast<f32x4_t*>(static_cast<float*>(out) + r * Nout + cfirst) =
                  f32x4_t{h[tt][0], h[tt][1], h[tt][2], h[tt][3]};
            } else {
              const uint32_t lo = f32_to_bf16_bits(h[tt][0]) | (f32_to_bf16_bits(h[tt][1]) << 16);
              const uint32_t hi = f32_to_bf16_bits(h[tt][2]) | (f32_to_bf16_bits(h[tt][3]) << 16);
              *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + r * Nout + cfirst) = make_uint2(lo, hi);
            }
          }
        }
      }
    } else if (kp == 0) {
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        const int c = chunk + tt * 16 + (lane & 15);
        if (c < nrows) {
          const size_t r = (size_t)(rows0 + c);
          *reinterpret_cast<f32x4_t*>(static_cast<float*>(out) + r * Nout + cfirst) = acc[0][tt];
        }
      }
    }
    __syncthreads();  // LDS is reused by the next chunk
  }
}

template <int DT, int FW, int KS, bool GATED, int OUT>
static hipError_t launch_tt(const FfnParams& p, int max_rows, int grid, hipStream_t stream) {
  const dim3 block(64 * FW * KS);
  if (max_rows <= 16)
    hipLaunchKernelGGL((ffn_kernel<DT, FW, KS, 1, GATED, OUT>), dim3(grid), block, 0, stream, p);
  else
    hipLaunchKernelGGL((ffn_kernel<DT, FW, KS, 2, GATED, OUT>), dim3(grid), block, 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_ffn(const FfnParams& p, int wdtype, bool gated, int out_dtype, int max_rows, int max_groups,
                      hipStream_t stream) {
  const long long grid = (long long)max_groups * p.tiles_r + (long long)p.n_shared * p.tiles_s;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  const int g = (int)grid;
  if (wdtype == MOE_F32) {
    if (gated) return launch_tt<MOE_F32, 1, 4, true, MOE_F32>(p, max_rows, g, stream);
    return launch_tt<MOE_F32, 1, 4, false, MOE_F32>(p, max_rows, g, stream);
  }
  if (wdtype == MOE_BF16) {
    if (gated) return launch_tt<MOE_BF16, 1, 4, true, MOE_BF16>(p, max_rows, g, stream);
    return launch_tt<MOE_BF16, 1, 4, false, MOE_F32>(p, max_rows, g, stream);
  }
  if (gated) return launch_tt<MOE_FP8_E4M3, 8, 1, true, MOE_FP8_E4M3>(p, max_rows, g, stream);
  (void)out_dtype;
  return launch_tt<MOE_FP8_E4M3, 1, 4, false, MOE_F32>(p, max_rows, g, stream);
}

}  // namespace moe
