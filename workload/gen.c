/*
 * Seeded synthetic inputs for MLA latent-cache decode.
 *
 * This module serves both the CPU oracle and the GPU library's tests and
 * benchmark. It holds no attention arithmetic: only random numbers, the
 * storage roundings of the input formats (bf16, fp16) and the cache writers
 * (q8_0, fp8, q4_0) that produce a quantized latent cache from float values.
 *
 * Random numbers come from one counter-based generator: output i of stream
 * (seed, stream) is the splitmix64 finaliser applied to key + (i+1)*gamma,
 * which is exactly the i-th output of a splitmix64 sequence started at
 * state = key (Steele, Lea, Flood, "Fast splittable pseudorandom number
 * generators", OOPSLA 2014). Any element can therefore be regenerated on its
 * own, and results do not depend on the number of threads.
 *
 * Normals use the Box-Muller transform on 24-bit uniforms in (0, 1]:
 * normal 2j uses the cosine branch and normal 2j+1 the sine branch of the
 * uniform pair (2j, 2j+1).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GEN_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

uint64_t gen_key(uint64_t seed, uint64_t stream) {
  return mix64(mix64(seed + GEN_GAMMA) ^ (stream * 0xD1B54A32D192ED03ULL));
}

static inline uint64_t gen_raw(uint64_t key, uint64_t i) {
  return mix64(key + (i + 1) * GEN_GAMMA);
}

/* 24-bit uniform in (0, 1]. */
static inline double gen_unif(uint64_t key, uint64_t i) {
  return (double)((gen_raw(key, i) >> 40) + 1) * (1.0 / 16777216.0);
}

static inline double gen_normal_at(uint64_t key, uint64_t i) {
  const uint64_t j = i >> 1;
  const double u1 = gen_unif(key, 2 * j);
  const double u2 = gen_unif(key, 2 * j + 1);
  const double r = sqrt(-2.0 * log(u1));
  const double a = 6.283185307179586476925 * u2;
  return (i & 1) ? r * sin(a) : r * cos(a);
}

/* float -> bf16 bits, round to nearest even (inputs here are finite). */
static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static inline float bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* float -> IEEE binary16 bits, round to nearest even, with subnormals. */
static uint16_t f32_to_fp16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  const uint32_t sign = (u >> 16) & 0x8000u;
  const uint32_t absu = u & 0x7FFFFFFFu;
  if (absu >= 0x7F800000u) /* inf or nan */
    return (uint16_t)(sign | 0x7C00u | (absu > 0x7F800000u ? 0x200u : 0u));
  const int e = (int)(absu >> 23) - 127; /* unbiased exponent */
  if (e > 15) return (uint16_t)(sign | 0x7C00u); /* overflow to inf */
  uint32_t mant = (absu & 0x7FFFFFu) | 0x800000u; /* 24-bit significand */
  int shift;                                      /* bits to drop from 24 */
  uint32_t exp_field;
  if (e >= -14) { /* normal half */
    shift = 13;
    exp_field = (uint32_t)(e + 15);
  } else { /* subnormal half: value = m * 2^-24 */
    if (absu == 0) return (uint16_t)sign;
    shift = 13 + (-14 - e);
    exp_field = 0;
    if (shift > 24) return (uint16_t)sign; /* rounds to zero */
  }
  uint32_t q = mant >> shift;
  const uint32_t rem = mant & ((1u << shift) - 1u);
  const uint32_t half = 1u << (shift - 1);
  if (rem > half || (rem == half && (q & 1u))) q += 1;
  uint32_t bits;
  if (exp_field == 0) {
    bits = q; /* may carry into the smallest normal, which is correct */
  } else {
    /* q holds the implicit bit at 2^10; a carry to 2^11 bumps the exponent */
    if (q >= 0x800u) {
      q >>= 1;
      exp_field += 1;
      if (exp_field >= 31) return (uint16_t)(sign | 0x7C00u);
    }
    bits = (exp_field << 10) | (q & 0x3FFu);
  }
  return (uint16_t)(sign | bits);
}

uint16_t gen_f32_to_bf16(float f) { return f32_to_bf16_rne(f); }
uint16_t gen_f32_to_fp16(float f) { return f32_to_fp16_rne(f); }
uint64_t gen_raw_at(uint64_t seed, uint64_t stream, uint64_t i) {
  return gen_raw(gen_key(seed, stream), i);
}
double gen_normal_value(uint64_t seed, uint64_t stream, uint64_t i) {
  return gen_normal_at(gen_key(seed, stream), i);
}

/* dst[k] = bf16(float(stddev * normal(offset + k))). */
void gen_normal_bf16(uint16_t* dst, int64_t n, uint64_t seed, uint64_t stream,
                     int64_t offset, double stddev) {
  const uint64_t key = gen_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t k = 0; k < n; ++k)
    dst[k] = f32_to_bf16_rne((float)(stddev * gen_normal_at(key, (uint64_t)(offset + k))));
}

void gen_normal_f32(float* dst, int64_t n, uint64_t seed, uint64_t stream,
                    int64_t offset, double stddev) {
  const uint64_t key = gen_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t k = 0; k < n; ++k)
    dst[k] = (float)(stddev * gen_normal_at(key, (uint64_t)(offset + k)));
}

void gen_normal_f64(double* dst, int64_t n, uint64_t seed, uint64_t stream,
                    int64_t offset, double stddev) {
  const uint64_t key = gen_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t k = 0; k < n; ++k)
    dst[k] = stddev * gen_normal_at(key, (uint64_t)(offset + k));
}

/* Integers uniform on [lo, hi] (inclusive). */
void gen_uniform_int(int32_t* dst, int64_t n, uint64_t seed, uint64_t stream,
                     int32_t lo, int32_t hi) {
  const uint64_t key = gen_key(seed, stream);
  const uint64_t span = (uint64_t)((int64_t)hi - (int64_t)lo + 1);
  for (int64_t k = 0; k < n; ++k)
    dst[k] = (int32_t)((int64_t)lo + (int64_t)(gen_raw(key, (uint64_t)k) % span));
}

/* Fisher-Yates shuffle of 0..n-1: for i = n-1 down to 1 swap perm[i] with
 * perm[j], j = raw(n-1-i) mod (i+1). */
void gen_permutation(int32_t* perm, int64_t n, uint64_t seed, uint64_t stream) {
  const uint64_t key = gen_key(seed, stream);
  for (int64_t i = 0; i < n; ++i) perm[i] = (int32_t)i;
  for (int64_t i = n - 1; i >= 1; --i) {
    const int64_t j = (int64_t)(gen_raw(key, (uint64_t)(n - 1 - i)) % (uint64_t)(i + 1));
    const int32_t t = perm[i];
    perm[i] = perm[j];
    perm[j] = t;
  }
}

/* mask[k] = 1 with probability p (uniform(k) <= p). */
void gen_bernoulli(uint8_t* mask, int64_t n, uint64_t seed, uint64_t stream, double p) {
  const uint64_t key = gen_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t k = 0; k < n; ++k) mask[k] = gen_unif(key, (uint64_t)k) <= p ? 1 : 0;
}

/* Multiply whole bf16 rows by an exact power-of-two factor where mask is set. */
void gen_scale_rows_bf16(uint16_t* rows, int64_t n_rows, int64_t row_len,
                         const uint8_t* mask, float factor) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n_rows; ++r) {
    if (!mask[r]) continue;
    uint16_t* p = rows + r * row_len;
    for (int64_t c = 0; c < row_len; ++c) p[c] = f32_to_bf16_rne(bf16_to_f32(p[c]) * factor);
  }
}

/*
 * q8_0-style cache writer: each row of `cols` floats (cols a multiple of 32)
 * is cut into groups of 32; per group a = max|x|, d = a / 127 (float),
 * q = clamp(round-half-away(x / d), -127, 127), and the stored scale is the
 * fp16 rounding of d. a == 0 gives d = 0 and q = 0.
 * Outputs: q [rows, cols] int8 and d16 [rows, cols / 32] fp16 bits.
 */
void gen_quantize_q8_0(const float* x, int64_t rows, int32_t cols, int8_t* q, uint16_t* d16) {
  const int32_t groups = cols / 32;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    for (int32_t g = 0; g < groups; ++g) {
      const float* xs = x + r * cols + g * 32;
      float amax = 0.0f;
      for (int k = 0; k < 32; ++k) {
        const float a = fabsf(xs[k]);
        if (a > amax) amax = a;
      }
      const float d = amax / 127.0f;
      d16[r * groups + g] = f32_to_fp16_rne(d);
      int8_t* qs = q + r * cols + g * 32;
      for (int k = 0; k < 32; ++k) {
        float v = d > 0.0f ? xs[k] / d : 0.0f;
        v = roundf(v); /* half away from zero */
        if (v > 127.0f) v = 127.0f;
        if (v < -127.0f) v = -127.0f;
        qs[k] = (int8_t)v;
      }
    }
  }
}

/*
 * fp8 cache writer: each row of 576 floats gets one fp32 scale
 * d = max |x| / 448 and codes E4M3(x / d), OCP E4M3 (bias 7, 3 fraction bits,
 * largest finite 448, no infinities) rounded to nearest even and saturated;
 * d = 0 for a row of zeros (codes 0).
 */
static uint8_t f32_to_e4m3_rne(float f) {
  const uint8_t sign = signbit(f) ? 0x80 : 0;
  const float a = fabsf(f);
  if (a < 0.015625f) return sign | (uint8_t)rintf(a * 512.0f);   /* steps of 2^-9 */
  int ex;
  frexpf(a, &ex);
  int e = ex - 1;
  float m = rintf(ldexpf(a, 3 - e));
  if (m >= 16.0f) {
    m = 8.0f;
    ++e;
  }
  if (e > 8) return sign | 0x7E;
  uint8_t code = (uint8_t)(((e + 7) << 3) | ((int)m - 8));
  return sign | (code == 0x7F ? 0x7E : code);
}

void gen_quantize_fp8(const float* x, int64_t rows, int32_t cols, uint8_t* q, float* scale) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    const float* xs = x + r * cols;
    float amax = 0.0f;
    for (int32_t k = 0; k < cols; ++k)
      if (fabsf(xs[k]) > amax) amax = fabsf(xs[k]);
    const float d = amax / 448.0f;
    scale[r] = d;
    for (int32_t k = 0; k < cols; ++k) q[r * cols + k] = d > 0.0f ? f32_to_e4m3_rne(xs[k] / d) : 0;
  }
}

/*
 * q4_0 block writer: every 32 floats get one fp16 scale d = m / -8 (m the
 * first value of largest magnitude) and 4-bit codes min(15, floor(x / d + 8.5))
 * (all 8 when d = 0), two per byte (code j of block g in byte 16 g + j / 2,
 * low nibble for even j). The values it is given stand for the rotated
 * blocks of a cache stored in Hadamard rotation: the rotation of independent
 * normal values is again independent normal values, so the generator draws
 * the rotated values directly and never rotates anything.
 */
void gen_quantize_q4_0(const float* x, int64_t rows, int32_t cols, uint8_t* q, uint16_t* d16) {
  const int32_t groups = cols / 32;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    for (int32_t g = 0; g < groups; ++g) {
      const float* xs = x + r * cols + g * 32;
      float m = 0.0f;
      for (int k = 0; k < 32; ++k)
        if (fabsf(xs[k]) > fabsf(m)) m = xs[k];
      const float d = m / -8.0f;
      d16[r * groups + g] = f32_to_fp16_rne(d);
      uint8_t* qs = q + r * (cols / 2) + g * 16;
      for (int k = 0; k < 32; k += 2) {
        int c[2];
        for (int h = 0; h < 2; ++h) {
          const float t = d != 0.0f ? floorf(xs[k + h] / d + 8.5f) : 8.0f;
          c[h] = t > 15.0f ? 15 : (int)t;
        }
        qs[k / 2] = (uint8_t)(c[0] | (c[1] << 4));
      }
    }
  }
}
