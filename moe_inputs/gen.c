/*
 * Seeded, counter-based input generator shared by the tests, the benchmark
 * and the oracle's callers.  It draws synthetic tensors only: it holds none
 * of the MoE layer's arithmetic.
 *
 * Every value is a pure function of (seed, tensor_id, index), so any thread
 * count, any chunking and any sub-range (one expert's weights, one token's
 * row) reproduce the same bytes.
 *
 * Random bits: SplitMix64 (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014).  The i-th output of a stream
 * with state s is mix64(s + (i + 1) * GAMMA).  The stream state of a tensor is
 * mix64(mix64(seed) ^ (tensor_id * C_TENSOR)).
 *
 * Normals: Box-Muller (1958) on two 24-bit uniforms taken from one 64-bit
 * output, evaluated in single precision (glibc logf / cosf / sqrtf), cosine
 * branch only; mean and std are applied in double.
 *
 * Storage rounding: fp32 -> bf16 is round-to-nearest-even on the bit pattern.
 * fp8 weight blocks (offline model preparation, not the layer's hot path):
 * per 128 x 128 block, scale = amax / 448 in fp32 (1 when amax is 0), and the
 * code is the OCP E4M3FN value nearest to w / scale, ties to the even code,
 * found by bisection over the 127 non-negative finite codes.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL
#define C_TENSOR 0xD1B54A32D192ED03ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t stream_state(uint64_t seed, uint64_t tensor_id) {
  return mix64(mix64(seed) ^ (tensor_id * C_TENSOR));
}

static inline uint64_t draw(uint64_t state, uint64_t index) {
  return mix64(state + (index + 1ULL) * GAMMA);
}

static inline double normal_from_bits(uint64_t r) {
  const float inv24 = 1.0f / 16777216.0f;
  float u1 = ((float)(r >> 40) + 0.5f) * inv24;
  float u2 = ((float)((r >> 16) & 0xFFFFFFULL) + 0.5f) * inv24;
  return (double)(sqrtf(-2.0f * logf(u1)) * cosf(6.28318530717958647692f * u2));
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

/* Uniform 64-bit draws (raw). */
void gen_bits(uint64_t seed, uint64_t tensor_id, uint64_t offset, int64_t n, uint64_t* out) {
  uint64_t s = stream_state(seed, tensor_id);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = draw(s, offset + (uint64_t)i);
}

/* mean + std * N(0,1), rounded to fp32. */
void gen_normal_f32(uint64_t seed, uint64_t tensor_id, uint64_t offset, int64_t n, double mean,
                    double std, float* out) {
  uint64_t s = stream_state(seed, tensor_id);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i)
    out[i] = (float)(mean + std * normal_from_bits(draw(s, offset + (uint64_t)i)));
}

/* Same values as gen_normal_f32, then rounded to bf16 (bit patterns). */
void gen_normal_bf16(uint64_t seed, uint64_t tensor_id, uint64_t offset, int64_t n, double mean,
                     double std, uint16_t* out) {
  uint64_t s = stream_state(seed, tensor_id);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i)
    out[i] = f32_to_bf16_rne((float)(mean + std * normal_from_bits(draw(s, offset + (uint64_t)i))));
}

/* Values of the non-negative finite E4M3FN codes 0..126: exponent bias 7,
 * 3 mantissa bits, subnormal step 2^-9, largest finite 448. */
static double e4m3_table[127];
static int e4m3_table_ready = 0;

static void e4m3_table_init(void) {
  if (e4m3_table_ready) return;
  for (int c = 0; c < 127; ++c) {
    int e = (c >> 3) & 15, m = c & 7;
    e4m3_table[c] = e == 0 ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
  }
  e4m3_table_ready = 1;
}

static uint8_t e4m3_encode_nearest(float v) {
  uint8_t sign = 0;
  double a = (double)v;
  if (a < 0) { sign = 0x80; a = -a; }
  if (a >= 448.0) return sign | 0x7E;
  int lo = 0, hi = 126; /* table[lo] <= a < table[hi] */
  while (hi - lo > 1) {
    int mid = (lo + hi) / 2;
    if (e4m3_table[mid] <= a) lo = mid; else hi = mid;
  }
  double dl = a - e4m3_table[lo], dh = e4m3_table[hi] - a;
  int c;
  if (dl < dh) c = lo;
  else if (dh < dl) c = hi;
  else c = (lo & 1) ? hi : lo;
  if (c == 0) return 0; /* +0 for any rounding to zero */
  return sign | (uint8_t)c;
}

/*
 * fp8 weight matrix [rows][cols] (rows % 128 == 0, cols % 128 == 0) whose
 * underlying values are mean + std * N(0,1) drawn at index
 * offset + r * cols + c of the stream, encoded per 128 x 128 block.
 * codes: [rows][cols] bytes; scales: [rows/128][cols/128] fp32.
 */
void gen_fp8_blocks(uint64_t seed, uint64_t tensor_id, uint64_t offset, int64_t rows, int64_t cols,
                    double mean, double std, uint8_t* codes, float* scales) {
  uint64_t s = stream_state(seed, tensor_id);
  int64_t rb = rows / 128, cb = cols / 128;
  e4m3_table_init();
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t b = 0; b < rb * cb; ++b) {
    int64_t br = b / cb, bc = b % cb;
    float vals[128 * 128];
    float amax = 0.f;
    for (int i = 0; i < 128; ++i)
      for (int j = 0; j < 128; ++j) {
        uint64_t idx = offset + (uint64_t)((br * 128 + i) * cols + bc * 128 + j);
        float v = (float)(mean + std * normal_from_bits(draw(s, idx)));
        vals[i * 128 + j] = v;
        float a = fabsf(v);
        if (a > amax) amax = a;
      }
    float scale = amax > 0.f ? amax / 448.0f : 1.0f;
    scales[b] = scale;
    for (int i = 0; i < 128; ++i)
      for (int j = 0; j < 128; ++j)
        codes[(br * 128 + i) * cols + bc * 128 + j] = e4m3_encode_nearest(vals[i * 128 + j] / scale);
  }
}

/* Seeded uniform permutation of 0..n-1 (Fisher-Yates, draw i picks among the
 * first n - i slots with a 64-bit multiply-shift, Lemire 2019 without the
 * rejection step; the bias is below 2^-50 for n < 2^14). */
void gen_permutation(uint64_t seed, uint64_t tensor_id, int32_t n, int32_t* out) {
  uint64_t s = stream_state(seed, tensor_id);
  for (int32_t i = 0; i < n; ++i) out[i] = i;
  for (int32_t i = n - 1; i > 0; --i) {
    uint64_t r = draw(s, (uint64_t)(n - 1 - i));
    int32_t j = (int32_t)(((unsigned __int128)r * (unsigned __int128)(uint64_t)(i + 1)) >> 64);
    int32_t t = out[i];
    out[i] = out[j];
    out[j] = t;
  }
}
