// Device-side helpers shared by the MoE kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr int kWave = 64;

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4_t;

// ---------------------------------------------------------------------------
// Storage conversions
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16, round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (u >> 16) | 0x40u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// fp32 -> OCP E4M3FN code, round to nearest even, saturating to +-448
// (|q| >= 448 gives 448; NaN gives the NaN code 0x7F).  Written from the format
// definition: exponent bias 7, 3 mantissa bits, subnormals are m * 2^-9.
__device__ __forceinline__ uint32_t f32_to_e4m3(float q) {
  uint32_t u = __float_as_uint(q);
  uint32_t sign = (u >> 24) & 0x80u;
  float a = fabsf(q);
  if (a != a) return 0x7Fu;
  if (a >= 448.0f) return sign | 0x7Eu;
  uint32_t code;
  if (a < 0.015625f) {                  // below 2^-6: subnormal step 2^-9
    code = (uint32_t)rintf(a * 512.0f);  // exact scaling, RNE; 8 is the first normal
  } else {
    uint32_t ua = __float_as_uint(a);
    int e = (int)((ua >> 23) & 0xFFu) - 127;  // -6 .. 8
    uint32_t mant = ua & 0x7FFFFFu;
    uint32_t m3 = mant >> 20, low = mant & 0xFFFFFu;
    if (low > 0x80000u || (low == 0x80000u && (m3 & 1u))) ++m3;
    if (m3 == 8u) { m3 = 0; ++e; }
    code = ((uint32_t)(e + 7) << 3) | m3;
  }
  return code == 0 ? 0u : (sign | code);
}

// ---------------------------------------------------------------------------
// Element traits: every GEMM streams rows in 256-byte steps; kStep elements.
// ---------------------------------------------------------------------------

template <int DT> struct Elem;
template <> struct Elem<MOE_F32> { static constexpr int kBytes = 4; static constexpr int kStep = 64; };
template <> struct Elem<MOE_BF16> { static constexpr int kBytes = 2; static constexpr int kStep = 128; };
template <> struct Elem<MOE_FP8_E4M3> { static constexpr int kBytes = 1; static constexpr int kStep = 256; };

// One lane's share of one 256-byte K-step of a 16-row tile: four 16-byte
// pieces.  Lane l (g = l / 16) holds bytes [64 q + 16 g, +16) of row l % 16
// for q = 0..3.  The MFMA operands below are built from these pieces; the A
// (weight) and B (activation) operands use the same piece -> k mapping, so
// the products sum over exactly the step's k values.
struct Step { i32x4_t q[4]; };

__device__ __forceinline__ void load_step(Step& s, const uint8_t* row_base, int lane) {
  const uint8_t* p = row_base + 16 * (lane >> 4);
#pragma unroll
  for (int q = 0; q < 4; ++q) s.q[q] = *reinterpret_cast<const i32x4_t*>(p + 64 * q);
}

__device__ __forceinline__ void zero_step(Step& s) {
#pragma unroll
  for (int q = 0; q < 4; ++q) s.q[q] = i32x4_t{0, 0, 0, 0};
}

// acc (16 x 16 fp32, lane layout of the 16x16 MFMAs) += A_step * B_step^T
template <int DT> struct Mma;

template <> struct Mma<MOE_BF16> {
  // v_mfma_f32_16x16x32_bf16: piece q holds k = 32 q + 8 g + 0..7.
  static __device__ __forceinline__ void run(f32x4_t& acc, const Step& a, const Step& b) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a.q[q]),
                                                    __builtin_bit_cast(bf16x8_t, b.q[q]), acc, 0, 0, 0);
  }
};

template <> struct Mma<MOE_F32> {
  // v_mfma_f32_16x16x4_f32: element e of piece q is k = 16 q + 4 g + e; one
  // MFMA per (q, e) reduces over the four lane groups.
  static __device__ __forceinline__ void run(f32x4_t& acc, const Step& a, const Step& b) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__int_as_float(a.q[q][e]), __int_as_float(b.q[q][e]),
                                                   acc, 0, 0, 0);
  }
};

// FP8: v_mfma_f32_16x16x128_f8f6f4 (E4M3 operands) per 128-k scale block h:
// pieces 2h and 2h+1 give lane group g the k values 128 h + 16 g + 0..15 and
// 128 h + 64 + 16 g + 0..15, i.e. the block is covered exactly once.
__device__ __forceinline__ f32x4_t mma_fp8_block(const Step& a, const Step& b, int h) {
  i32x8_t av, bv;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    av[i] = a.q[2 * h][i];
    av[4 + i] = a.q[2 * h + 1][i];
    bv[i] = b.q[2 * h][i];
    bv[4 + i] = b.q[2 * h + 1][i];
  }
  f32x4_t z = {0.f, 0.f, 0.f, 0.f};
  // format codes 0/0: both operands E4M3.  Zero scale operands select the
  // unscaled v_mfma_f32_16x16x128_f8f6f4 (block scales are applied outside).
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, z, 0, 0, 0, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Wave-level helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

}  // namespace moe
