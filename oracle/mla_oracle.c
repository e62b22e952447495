/*
 * CPU oracle for MLA latent-cache decode -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the package smoke check and the benchmark's CPU
 * baseline may load or call this file's library. The GPU library never
 * does, and shares no code with it.
 *
 * Everything is plain, slow, fp64 arithmetic taken from the definitions:
 *
 *  - MLA caches one latent vector c_KV per token instead of per-head keys and
 *    values, and recovers them with up-projections k = W_UK c, v = W_UV c
 *    ("MLA: Multi-Head Latent Attention -- DeepSeek-AI Explained", section
 *    Method, the three architecture equations).
 *  - The up-projections can be folded into the query and output projections,
 *    so attention runs directly against the latent ("Weight Absorbing
 *    Trick", nnets.ru article on MLA and FlashAttention, section on the
 *    essence of MLA; snowgate.dev forum thread 35, last reply: W_UK absorbed
 *    into the query).
 *  - Each cached row is the 512-wide latent plus a 64-wide decoupled RoPE key
 *    shared by all heads, which is kept as a separate slice so the absorption
 *    still holds (snowgate.dev thread 35, replies on the 512 + 64 row).
 *  - The kernel is a FlashAttention-style exact attention (FlashMLA page of
 *    the ik_llama.cpp docs, "What is MLA?"), so the reference is plain
 *    softmax attention computed directly in two passes.
 *  - The q8_0 cache type (FlashMLA page, "KV cache with MLA"): blocks of 32
 *    int8 values sharing one fp16 scale; a value is scale * int.
 *  - The low-bit cache with a Hadamard transform of the keys before
 *    quantisation (same page and section, the q4_0 cache with the K-cache
 *    Hadamard option): here every 32-value block of a row is rotated by the
 *    orthonormal 32-point Walsh-Hadamard matrix and stored as a q4_0 block
 *    (4-bit codes, one fp16 scale); reading it back rotates the block again.
 *
 * Readings where the pages are silent (the paged layout, the causal rule for
 * several new tokens, empty rows, the split plan) follow the API contract of
 * the GPU library and are spelled out at each function.
 *
 * Parity pins: every function here is pinned by CPU tests against closed
 * forms, invariants and brute force (absorbed == decompressed on random
 * W_UK / W_UV; uniform and one-hot softmax cases; exact rows; LSE combine of
 * a token partition == the unsplit result; IEEE binary16 / bfloat16 decoding
 * of chosen bit patterns; partition invariants of the plan).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define D_LATENT 512
#define D_ROPE 64
#define D_K (D_LATENT + D_ROPE)
#define BLOCK_TOKENS 64
#define Q8_GROUP 32
#define Q8_GROUPS (D_K / Q8_GROUP)
#define D_HEAD_NOPE 128 /* per-head no-RoPE key width of the decompressed form */
#define D_HEAD_V 128    /* per-head value width of the decompressed form */
#define Q4_ROW_BYTES (D_K / 2) /* q4_0 codes of one row, two per byte */

/* ------------------------------------------------------------ decoding */

/* bfloat16: the upper 16 bits of an IEEE binary32. Exact in double. */
double oracle_bf16_value(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* IEEE 754 binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double oracle_fp16_value(uint16_t bits) {
  const int s = bits >> 15;
  const int e = (bits >> 10) & 0x1F;
  const int m = bits & 0x3FF;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24); /* subnormal: m * 2^-24 */
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + m), e - 25); /* (1 + m/1024) * 2^(e-15) */
  return s ? -v : v;
}

/* q8_0 dequantization of one value: scale * int, exact in double. */
double oracle_q8_value(int8_t qv, uint16_t scale_bits) {
  return oracle_fp16_value(scale_bits) * (double)qv;
}

/* OCP 8-bit float E4M3 (the "fp8" of the forum's fp8 KV cache; 1 sign, 4
 * exponent bits with bias 7, 3 fraction bits, no infinities): exponent 0 is
 * subnormal (m/8 * 2^-6), S.1111.111 is NaN, the largest finite value is
 * 1.75 * 2^8 = 448. Exact in double. */
double oracle_fp8_value(uint8_t bits) {
  const int s = bits >> 7, e = (bits >> 3) & 0xF, m = bits & 7;
  double v;
  if (e == 15 && m == 7)
    v = NAN;
  else if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp((double)(8 + m), e - 10);
  return s ? -v : v;
}

/* E4M3 encoding of a finite float, rounded to nearest (ties to even) and
 * saturated to +-448 (the NaN code is never produced for a finite input). */
uint8_t oracle_fp8_bits(float f) {
  const uint8_t sign = signbit(f) ? 0x80 : 0;
  const double a = fabs((double)f);
  if (a < ldexp(1.0, -6)) {                  /* subnormal range: steps of 2^-9 */
    const double m = rint(ldexp(a, 9));      /* 0 .. 8; 8 is the smallest normal */
    return sign | (uint8_t)m;
  }
  int ex;
  frexp(a, &ex);                             /* a = f * 2^ex, f in [0.5, 1) */
  int E = ex - 1;
  double sig = rint(ldexp(a, 3 - E));        /* 8 .. 16 */
  if (sig >= 16.0) {
    sig = 8.0;
    ++E;
  }
  if (E > 8) return sign | 0x7E;
  uint8_t code = (uint8_t)(((E + 7) << 3) | (int)(sig - 8.0));
  if (code == 0x7F) code = 0x7E;             /* above 448: saturate */
  return sign | code;
}

/* fp8 cache writer for one row of 576 values: one fp32 scale per token,
 * d = max |x| / 448, stored as is; code = E4M3(x / d) (fp32 division); a row
 * of zeros gives d = 0 and codes 0. A cached value is d * E4M3 value. */
void oracle_quantize_fp8_row(const float* x, uint8_t* q, float* scale) {
  float amax = 0.0f;
  for (int d = 0; d < D_K; ++d)
    if (fabsf(x[d]) > amax) amax = fabsf(x[d]);
  const float dsc = amax / 448.0f;
  *scale = dsc;
  for (int d = 0; d < D_K; ++d) q[d] = dsc > 0.0f ? oracle_fp8_bits(x[d] / dsc) : 0;
}

/* Host threads the parallel loops below use (OpenMP), and a way to change it
 * (timing a single core). */
int oracle_max_threads(void) { return omp_get_max_threads(); }
void oracle_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }

/* IEEE 754 binary16 bits of a float, rounded to nearest (ties to even):
 * overflow to infinity from 65520 up (65504 plus half a unit in the last
 * place), subnormals below 2^-14 in steps of 2^-24. NaN gives 0x7E00. */
uint16_t oracle_fp16_bits(float f) {
  const double v0 = (double)f;
  if (isnan(v0)) return 0x7E00;
  const uint16_t sign = signbit(v0) ? 0x8000 : 0;
  const double v = fabs(v0);
  if (v >= 65520.0) return sign | 0x7C00;
  if (v < ldexp(1.0, -14)) {
    /* subnormal (or zero): v = m * 2^-24, m rounded to nearest even; m = 1024
     * is the smallest normal, whose bits are 0x0400 as well */
    const double m = rint(ldexp(v, 24));
    return sign | (uint16_t)m;
  }
  int ex;
  frexp(v, &ex);                     /* v = f * 2^ex, f in [0.5, 1) */
  int E = ex - 1;                    /* v = 1.x * 2^E */
  double sig = rint(ldexp(v, 10 - E));   /* in [1024, 2048] */
  if (sig >= 2048.0) {
    sig = 1024.0;
    ++E;
  }
  if (E + 15 >= 31) return sign | 0x7C00;
  return sign | (uint16_t)((E + 15) << 10) | (uint16_t)(sig - 1024.0);
}

/* q8_0 cache writer for one row of 576 values, the quantisation behind the
 * q8_0 cache type (FlashMLA page, "KV cache with MLA"): per group g of 32
 * columns, a = max |x|, d = a / 127 in fp32, stored scale fp16(d) (nearest
 * even), code = x / d (fp32) rounded half away from zero and clamped to
 * [-127, 127]; a = 0 gives scale 0 and codes 0. A cached value is then
 * fp16(d) * code. */
void oracle_quantize_q8_0_row(const float* x, int8_t* q, uint16_t* scales) {
  for (int g = 0; g < Q8_GROUPS; ++g) {
    const float* xs = x + g * Q8_GROUP;
    float amax = 0.0f;
    for (int k = 0; k < Q8_GROUP; ++k)
      if (fabsf(xs[k]) > amax) amax = fabsf(xs[k]);
    const float d = amax / 127.0f;
    scales[g] = oracle_fp16_bits(d);
    for (int k = 0; k < Q8_GROUP; ++k) {
      float c = 0.0f;
      if (d > 0.0f) {
        const float r = xs[k] / d;
        const float t = truncf(r);
        c = fabsf(r - t) >= 0.5f ? t + (r > 0.0f ? 1.0f : -1.0f) : t;
      }
      if (c > 127.0f) c = 127.0f;
      if (c < -127.0f) c = -127.0f;
      q[g * Q8_GROUP + k] = (int8_t)c;
    }
  }
}

/* --------------------------------------- q4_0 blocks in Hadamard rotation */

/*
 * The rotation. H is the 32 x 32 Sylvester-Hadamard matrix,
 * H[m][j] = (-1)^popcount(m & j); R = H / sqrt(32) is symmetric and
 * orthogonal, so R R = I and R is its own inverse. A cached row is stored
 * block by block (block g = columns 32g .. 32g+31) as the q4_0 encoding of
 * y = R x_g, and read back as x_g = R y.
 */
int oracle_hadamard_sign(int m, int j) { return (__builtin_popcount((unsigned)(m & j)) & 1) ? -1 : 1; }

/* y = R x for one block, in double, straight from the matrix entries. */
void oracle_hadamard32(const double* x, double* y) {
  for (int m = 0; m < Q8_GROUP; ++m) {
    double acc = 0.0;
    for (int j = 0; j < Q8_GROUP; ++j) acc += oracle_hadamard_sign(m, j) * x[j];
    y[m] = acc / sqrt((double)Q8_GROUP);
  }
}

/* Value of one cached q4_0 code: scale * (code - 8), exact in double. */
double oracle_q4_value(int code, uint16_t scale_bits) {
  return oracle_fp16_value(scale_bits) * (double)(code - 8);
}

/* Code j (0..31) of a 16-byte q4_0 block: byte j / 2, low nibble for even j. */
int oracle_q4_code(const uint8_t* blk, int j) { return (blk[j >> 1] >> (4 * (j & 1))) & 0xF; }

/*
 * The cache writer for one row of 576 values (the reading where the pages
 * name the format only). Per block, in single precision and in this order
 * (the decision that picks each integer code is taken in the precision and
 * order the GPU writer uses):
 *   1. y = R x by the fast Walsh-Hadamard transform: for s = 1, 2, 4, 8, 16,
 *      every pair (i, i + s) with i & s = 0 becomes (a + b, a - b); then each
 *      y times the single-precision value of 1/sqrt(32);
 *   2. q4_0: m = the first y of largest magnitude, d = m / -8,
 *      code = min(15, floor(y / d + 8.5)) (so m itself gets code 0), every
 *      code 8 when d = 0; the stored scale is fp16(d) (round to nearest even).
 * Codes go two per byte, code j of block g in byte 16 g + j / 2, low nibble
 * for even j.
 */
void oracle_quantize_q4h_row(const float* x, uint8_t* q, uint16_t* scales) {
  const float inv_sqrt32 = (float)(1.0 / sqrt(32.0));
  for (int g = 0; g < Q8_GROUPS; ++g) {
    float y[Q8_GROUP];
    for (int j = 0; j < Q8_GROUP; ++j) y[j] = x[g * Q8_GROUP + j];
    for (int st = 1; st < Q8_GROUP; st <<= 1)
      for (int i = 0; i < Q8_GROUP; ++i)
        if ((i & st) == 0) {
          const float a = y[i], b = y[i + st];
          y[i] = a + b;
          y[i + st] = a - b;
        }
    for (int j = 0; j < Q8_GROUP; ++j) y[j] = y[j] * inv_sqrt32;
    float m = 0.0f;
    for (int j = 0; j < Q8_GROUP; ++j)
      if (fabsf(y[j]) > fabsf(m)) m = y[j];
    const float d = m / -8.0f;
    scales[g] = oracle_fp16_bits(d);
    uint8_t* blk = q + 16 * g;
    for (int j = 0; j < Q8_GROUP; j += 2) {
      int c[2];
      for (int h = 0; h < 2; ++h) {
        if (d == 0.0f) {
          c[h] = 8;
        } else {
          const float t = floorf(y[j + h] / d + 8.5f);
          c[h] = t > 15.0f ? 15 : (int)t;
        }
      }
      blk[j >> 1] = (uint8_t)(c[0] | (c[1] << 4));
    }
  }
}

/* One cached row of a q4_0 cache in Hadamard rotation, read back: per block
 * the stored values scale * (code - 8), rotated back by R. */
void oracle_q4h_row(const uint8_t* codes, const uint16_t* scales, double* dst) {
  for (int g = 0; g < Q8_GROUPS; ++g) {
    double y[Q8_GROUP];
    for (int j = 0; j < Q8_GROUP; ++j) y[j] = oracle_q4_value(oracle_q4_code(codes + 16 * g, j), scales[g]);
    oracle_hadamard32(y, dst + Q8_GROUP * g);
  }
}

/* The same for `rows` consecutive rows (codes [rows, 288], scales [rows, 18],
 * out double [rows, 576]): the whole cache read back once, so that a decode
 * of a large workload can run over it as fp64 rows (cache kind 4) instead of
 * rotating every block back for every query row. */
void oracle_q4h_dequantize(int64_t rows, const uint8_t* codes, const uint16_t* scales,
                           double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    oracle_q4h_row(codes + r * Q4_ROW_BYTES, scales + r * Q8_GROUPS, out + r * D_K);
}

/* ------------------------------------------------------------ paged cache */

typedef struct {
  int kind; /* 0: bf16 bits, 1: q8_0, 2: fp8 with per-token fp32 scales, 3: q4_0 in
               Hadamard rotation, 4: fp64 rows */
  const void* kv;
  const void* scales;
  int64_t num_blocks;
  const int32_t* block_table;
  int32_t max_blocks;
} cache_view;

/* Token t of a sequence lives in row t % 64 of physical block
 * block_table[b][t / 64]. Writes its 576 values (exactly) to dst. */
static void cache_row(const cache_view* c, int32_t b, int64_t t, double* dst) {
  const int64_t phys = c->block_table[(int64_t)b * c->max_blocks + t / BLOCK_TOKENS];
  const int64_t row = phys * BLOCK_TOKENS + t % BLOCK_TOKENS;
  if (c->kind == 0) {
    const uint16_t* r = (const uint16_t*)c->kv + row * D_K;
    for (int d = 0; d < D_K; ++d) dst[d] = oracle_bf16_value(r[d]);
  } else if (c->kind == 1) {
    const int8_t* r = (const int8_t*)c->kv + row * D_K;
    const uint16_t* s = (const uint16_t*)c->scales + row * Q8_GROUPS;
    for (int d = 0; d < D_K; ++d) dst[d] = oracle_q8_value(r[d], s[d / Q8_GROUP]);
  } else if (c->kind == 2) {
    const uint8_t* r = (const uint8_t*)c->kv + row * D_K;
    const double s = (double)((const float*)c->scales)[row];
    for (int d = 0; d < D_K; ++d) dst[d] = s * oracle_fp8_value(r[d]);
  } else if (c->kind == 3) {
    oracle_q4h_row((const uint8_t*)c->kv + row * Q4_ROW_BYTES,
                   (const uint16_t*)c->scales + row * Q8_GROUPS, dst);
  } else {
    /* rows given as doubles (a cache read back once, e.g. by
       oracle_q4h_dequantize, for large workloads) */
    memcpy(dst, (const double*)c->kv + row * D_K, sizeof(double) * D_K);
  }
}

/* Tokens of sequence b after clamping its length to the table's capacity;
 * negative lengths count as empty. */
static int64_t seq_tokens(const int32_t* seqlens, int32_t b, int32_t max_blocks) {
  int64_t L = seqlens[b];
  if (L < 0) L = 0;
  if (L > (int64_t)max_blocks * BLOCK_TOKENS) L = (int64_t)max_blocks * BLOCK_TOKENS;
  return L;
}

/* A sequence is valid when every block it uses has an id in [0, num_blocks).
 * Invalid sequences produce NaN output and NaN lse for all their rows. */
static int seq_valid(const cache_view* c, int32_t b, int64_t L) {
  const int64_t nb = (L + BLOCK_TOKENS - 1) / BLOCK_TOKENS;
  for (int64_t j = 0; j < nb; ++j) {
    const int32_t id = c->block_table[(int64_t)b * c->max_blocks + j];
    if (id < 0 || (int64_t)id >= c->num_blocks) return 0;
  }
  return 1;
}

/* Visible tokens of query i among s_q new tokens: the cache length L already
 * includes the new tokens, and query i sees positions 0 .. L - s_q + i. */
static int64_t visible_tokens(int64_t L, int32_t s_q, int32_t i) {
  const int64_t n = L - s_q + 1 + i;
  return n > 0 ? n : 0;
}

/* ------------------------------------------------- absorbed latent attention */

/*
 * One query row against the latent cache, two passes:
 *   s_t   = scale * sum_{d<576} q[d] * r_t[d]       (t < n)
 *   m     = max_t s_t,   l = sum_t exp(s_t - m),   lse = m + ln l
 *   out_e = sum_t exp(s_t - m) * r_t[e] / l        (e < 512: V is the latent)
 * n == 0 gives out = 0 and lse = -inf.
 */
static void absorbed_row(const cache_view* c, int32_t b, int64_t n, const double* q,
                         double scale, double* out, double* lse, double* s, double* row,
                         double* out_abs) {
  for (int e = 0; e < D_LATENT; ++e) out[e] = 0.0;
  if (out_abs)
    for (int e = 0; e < D_LATENT; ++e) out_abs[e] = 0.0;
  if (n == 0) {
    *lse = -INFINITY;
    return;
  }
  double m = -INFINITY;
  for (int64_t t = 0; t < n; ++t) {
    cache_row(c, b, t, row);
    double acc = 0.0;
    for (int d = 0; d < D_K; ++d) acc += q[d] * row[d];
    s[t] = scale * acc;
    if (s[t] > m) m = s[t];
  }
  double l = 0.0;
  for (int64_t t = 0; t < n; ++t) {
    const double p = exp(s[t] - m);
    l += p;
    cache_row(c, b, t, row);
    for (int e = 0; e < D_LATENT; ++e) out[e] += p * row[e];
    if (out_abs)
      for (int e = 0; e < D_LATENT; ++e) out_abs[e] += p * fabs(row[e]);
  }
  for (int e = 0; e < D_LATENT; ++e) out[e] /= l;
  if (out_abs)
    for (int e = 0; e < D_LATENT; ++e) out_abs[e] /= l;
  *lse = m + log(l);
}

static int decode_absorbed_core(int32_t B, int32_t s_q, int32_t H, const uint16_t* q_bf16,
                                const double* q_f64, const cache_view* c,
                                const int32_t* seqlens, double scale, const int64_t* rows,
                                int64_t n_rows, double* out, double* lse, double* out_abs) {
  const int64_t total = (int64_t)B * s_q * H;
  if (!rows) n_rows = total;
  int err = 0;
#pragma omp parallel
  {
    double* row = (double*)malloc(sizeof(double) * D_K);
    double* qrow = (double*)malloc(sizeof(double) * D_K);
    double* s = NULL;
    int64_t s_cap = 0;
#pragma omp for schedule(dynamic, 1)
    for (int64_t k = 0; k < n_rows; ++k) {
      const int64_t r = rows ? rows[k] : k;
      double* o = out + k * D_LATENT;
      if (r < 0 || r >= total) {
#pragma omp atomic write
        err = 1;
        continue;
      }
      const int32_t i = (int32_t)((r / H) % s_q);
      const int32_t b = (int32_t)(r / ((int64_t)H * s_q));
      const int64_t L = seq_tokens(seqlens, b, c->max_blocks);
      double* oa = out_abs ? out_abs + k * D_LATENT : NULL;
      if (!seq_valid(c, b, L)) {
        for (int e = 0; e < D_LATENT; ++e) o[e] = NAN;
        if (oa)
          for (int e = 0; e < D_LATENT; ++e) oa[e] = NAN;
        lse[k] = NAN;
        continue;
      }
      const int64_t n = visible_tokens(L, s_q, i);
      if (n > s_cap) {
        free(s);
        s = (double*)malloc(sizeof(double) * (size_t)n);
        s_cap = n;
      }
      for (int d = 0; d < D_K; ++d)
        qrow[d] = q_bf16 ? oracle_bf16_value(q_bf16[r * D_K + d]) : q_f64[r * D_K + d];
      absorbed_row(c, b, n, qrow, scale, o, &lse[k], s, row, oa);
    }
    free(row);
    free(qrow);
    free(s);
  }
  return err ? -1 : 0;
}

/*
 * Absorbed-form decode, the contract of the GPU kernel.
 *   q          bf16 bits [B, s_q, H, 576], row r = (b * s_q + i) * H + h
 *   kv         bf16 bits, int8 or fp8 [num_blocks, 64, 576] (kv_kind 0 / 1 / 2),
 *              q4_0 codes [num_blocks, 64, 288] in Hadamard rotation (kv_kind 3),
 *              or double [num_blocks, 64, 576] (kv_kind 4, the rows themselves)
 *   kv_scales  fp16 bits [num_blocks, 64, 18] for q8_0 and q4_0, fp32
 *              [num_blocks, 64] for fp8, else NULL
 *   block_table int32 [B, max_blocks]; seqlens int32 [B] (new tokens included)
 *   rows       optional list of row ids to compute (NULL = all, in order)
 *   out        double [n_rows, 512];  lse double [n_rows] (natural log)
 * Returns 0, or -1 if a row id is out of range.
 */
int oracle_decode_absorbed(int32_t B, int32_t s_q, int32_t H, const uint16_t* q,
                           int32_t kv_kind, const void* kv, const void* kv_scales,
                           int64_t num_blocks, const int32_t* block_table, int32_t max_blocks,
                           const int32_t* seqlens, double softmax_scale, const int64_t* rows,
                           int64_t n_rows, double* out, double* lse) {
  cache_view c = {kv_kind, kv, kv_scales, num_blocks, block_table, max_blocks};
  return decode_absorbed_core(B, s_q, H, q, NULL, &c, seqlens, softmax_scale, rows, n_rows,
                              out, lse, NULL);
}

/* Same, plus out_abs [n_rows, 512] = sum_t p_t |r_t[e]|: the magnitude of the
 * terms behind each output value. Rounding the probabilities (or the output)
 * to a format with relative precision u perturbs out[e] by at most about
 * u * out_abs[e], which is what an error bound for such arithmetic scales
 * with; out_abs >= |out| always, with equality when all terms share a sign. */
int oracle_decode_absorbed_abs(int32_t B, int32_t s_q, int32_t H, const uint16_t* q,
                               int32_t kv_kind, const void* kv, const void* kv_scales,
                               int64_t num_blocks, const int32_t* block_table,
                               int32_t max_blocks, const int32_t* seqlens, double softmax_scale,
                               const int64_t* rows, int64_t n_rows, double* out, double* lse,
                               double* out_abs) {
  cache_view c = {kv_kind, kv, kv_scales, num_blocks, block_table, max_blocks};
  return decode_absorbed_core(B, s_q, H, q, NULL, &c, seqlens, softmax_scale, rows, n_rows,
                              out, lse, out_abs);
}

/* Same, with an fp64 query [B, s_q, H, 576] (used for the absorption check). */
int oracle_decode_absorbed_f64q(int32_t B, int32_t s_q, int32_t H, const double* q,
                                int32_t kv_kind, const void* kv, const void* kv_scales,
                                int64_t num_blocks, const int32_t* block_table,
                                int32_t max_blocks, const int32_t* seqlens,
                                double softmax_scale, double* out, double* lse) {
  cache_view c = {kv_kind, kv, kv_scales, num_blocks, block_table, max_blocks};
  return decode_absorbed_core(B, s_q, H, NULL, q, &c, seqlens, softmax_scale, NULL, 0, out,
                              lse, NULL);
}

/* ------------------------------------------------------------ cache append */

/*
 * Appending the new tokens of a decode step to the paged cache: the s_q new
 * rows of sequence b are its last s_q tokens, so new row i lands at position
 * t = L_b - s_q + i (L_b = seqlens[b], which already counts them), i.e. in row
 * t % 64 of physical block block_table[b][t / 64]. Positions outside
 * [0, 64 * max_blocks) and blocks outside [0, num_blocks) are skipped.
 *   rows   bf16 bits [B, s_q, 576]: the new [c_KV | k_rope] rows
 *   kind 0: kv bf16 bits [num_blocks, 64, 576], written as given;
 *   kind 1: kv int8 [num_blocks, 64, 576] + scales fp16 bits [num_blocks, 64, 18],
 *           written by the q8_0 cache writer above;
 *   kind 2: kv fp8 [num_blocks, 64, 576] + scales fp32 [num_blocks, 64], written by
 *           the fp8 cache writer above;
 *   kind 3: kv uint8 [num_blocks, 64, 288] (q4_0 codes) + scales fp16 bits
 *           [num_blocks, 64, 18], written by the rotating q4_0 writer above.
 * Returns the number of rows written.
 */
int64_t oracle_cache_append(int32_t B, int32_t s_q, int32_t kind, const uint16_t* rows,
                            const int32_t* block_table, int32_t max_blocks,
                            const int32_t* seqlens, int64_t num_blocks, void* kv,
                            void* scales) {
  int64_t written = 0;
  float x[D_K];
  for (int32_t b = 0; b < B; ++b) {
    for (int32_t i = 0; i < s_q; ++i) {
      const int64_t t = (int64_t)seqlens[b] - s_q + i;
      if (t < 0 || t >= (int64_t)max_blocks * BLOCK_TOKENS) continue;
      const int32_t blk = block_table[(int64_t)b * max_blocks + t / BLOCK_TOKENS];
      if (blk < 0 || (int64_t)blk >= num_blocks) continue;
      const int64_t dst = (int64_t)blk * BLOCK_TOKENS + t % BLOCK_TOKENS;
      const uint16_t* src = rows + ((int64_t)b * s_q + i) * D_K;
      if (kind == 0) {
        memcpy((uint16_t*)kv + dst * D_K, src, sizeof(uint16_t) * D_K);
      } else {
        for (int d = 0; d < D_K; ++d) x[d] = (float)oracle_bf16_value(src[d]);
        if (kind == 1)
          oracle_quantize_q8_0_row(x, (int8_t*)kv + dst * D_K, (uint16_t*)scales + dst * Q8_GROUPS);
        else if (kind == 2)
          oracle_quantize_fp8_row(x, (uint8_t*)kv + dst * D_K, (float*)scales + dst);
        else
          oracle_quantize_q4h_row(x, (uint8_t*)kv + dst * Q4_ROW_BYTES,
                                  (uint16_t*)scales + dst * Q8_GROUPS);
      }
      ++written;
    }
  }
  return written;
}

/* ------------------------------------------ decompressed (non-absorbed) form */

/*
 * The definition without absorption: per head h and visible token t,
 *   k_{t,h} = [ W_UK[h] c_t ; k_rope_t ]   (128 + 64 wide)
 *   v_{t,h} =   W_UV[h] c_t                (128 wide)
 * with c_t = r_t[0:512], k_rope_t = r_t[512:576], then standard softmax
 * attention of q_h = [q_nope_h ; q_rope_h] and the per-head output
 * o_h = sum_t p_t v_{t,h}.
 *   q_nope [B, s_q, H, 128], q_rope [B, s_q, H, 64] (fp64)
 *   w_uk, w_uv [H, 128, 512] (fp64, row j of W is the j-th output dim)
 *   out [B, s_q, H, 128], lse [B, s_q, H]
 */
int oracle_decode_decompressed(int32_t B, int32_t s_q, int32_t H, const double* q_nope,
                               const double* q_rope, const double* w_uk, const double* w_uv,
                               const uint16_t* kv, int64_t num_blocks,
                               const int32_t* block_table, int32_t max_blocks,
                               const int32_t* seqlens, double softmax_scale, double* out,
                               double* lse) {
  cache_view c = {0, kv, NULL, num_blocks, block_table, max_blocks};
  const int64_t total = (int64_t)B * s_q * H;
#pragma omp parallel
  {
    double* row = (double*)malloc(sizeof(double) * D_K);
    double* v = (double*)malloc(sizeof(double) * D_HEAD_V);
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < total; ++r) {
      const int32_t h = (int32_t)(r % H);
      const int32_t i = (int32_t)((r / H) % s_q);
      const int32_t b = (int32_t)(r / ((int64_t)H * s_q));
      const double* qn = q_nope + r * D_HEAD_NOPE;
      const double* qr = q_rope + r * D_ROPE;
      const double* wk = w_uk + (int64_t)h * D_HEAD_NOPE * D_LATENT;
      const double* wv = w_uv + (int64_t)h * D_HEAD_V * D_LATENT;
      double* o = out + r * D_HEAD_V;
      const int64_t L = seq_tokens(seqlens, b, max_blocks);
      for (int j = 0; j < D_HEAD_V; ++j) o[j] = 0.0;
      if (!seq_valid(&c, b, L)) {
        for (int j = 0; j < D_HEAD_V; ++j) o[j] = NAN;
        lse[r] = NAN;
        continue;
      }
      const int64_t n = visible_tokens(L, s_q, i);
      if (n == 0) {
        lse[r] = -INFINITY;
        continue;
      }
      double* s = (double*)malloc(sizeof(double) * (size_t)n);
      double m = -INFINITY;
      for (int64_t t = 0; t < n; ++t) {
        cache_row(&c, b, t, row);
        double acc = 0.0;
        for (int j = 0; j < D_HEAD_NOPE; ++j) {
          double k = 0.0;
          for (int d = 0; d < D_LATENT; ++d) k += wk[j * D_LATENT + d] * row[d];
          acc += qn[j] * k;
        }
        for (int d = 0; d < D_ROPE; ++d) acc += qr[d] * row[D_LATENT + d];
        s[t] = softmax_scale * acc;
        if (s[t] > m) m = s[t];
      }
      double l = 0.0;
      for (int64_t t = 0; t < n; ++t) {
        const double p = exp(s[t] - m);
        l += p;
        cache_row(&c, b, t, row);
        for (int j = 0; j < D_HEAD_V; ++j) {
          double vj = 0.0;
          for (int d = 0; d < D_LATENT; ++d) vj += wv[j * D_LATENT + d] * row[d];
          v[j] = vj;
        }
        for (int j = 0; j < D_HEAD_V; ++j) o[j] += p * v[j];
      }
      for (int j = 0; j < D_HEAD_V; ++j) o[j] /= l;
      lse[r] = m + log(l);
      free(s);
    }
    free(row);
    free(v);
  }
  return 0;
}

/* Absorbed query: q~_h = [ W_UK[h]^T q_nope_h ; q_rope_h ]  -> [rows, 576],
 * since q_nope . (W_UK c) = (W_UK^T q_nope) . c. */
void oracle_absorb_query(int64_t rows, int32_t H, const double* q_nope, const double* q_rope,
                         const double* w_uk, double* q_abs) {
  for (int64_t r = 0; r < rows; ++r) {
    const int32_t h = (int32_t)(r % H);
    const double* wk = w_uk + (int64_t)h * D_HEAD_NOPE * D_LATENT;
    double* qa = q_abs + r * D_K;
    for (int d = 0; d < D_LATENT; ++d) {
      double acc = 0.0;
      for (int j = 0; j < D_HEAD_NOPE; ++j) acc += wk[j * D_LATENT + d] * q_nope[r * D_HEAD_NOPE + j];
      qa[d] = acc;
    }
    for (int d = 0; d < D_ROPE; ++d) qa[D_LATENT + d] = q_rope[r * D_ROPE + d];
  }
}

/* Per-head output from the latent-space output: o_h = W_UV[h] o_lat_h. */
void oracle_project_output(int64_t rows, int32_t H, const double* o_lat, const double* w_uv,
                           double* o) {
  for (int64_t r = 0; r < rows; ++r) {
    const int32_t h = (int32_t)(r % H);
    const double* wv = w_uv + (int64_t)h * D_HEAD_V * D_LATENT;
    for (int j = 0; j < D_HEAD_V; ++j) {
      double acc = 0.0;
      for (int d = 0; d < D_LATENT; ++d) acc += wv[j * D_LATENT + d] * o_lat[r * D_LATENT + d];
      o[r * D_HEAD_V + j] = acc;
    }
  }
}

/* --------------------------------------------------------- LSE combine */

/*
 * Merge S partial results of the same rows computed over disjoint token
 * sets:  lse = ln sum_s exp(lse_s),  out = sum_s exp(lse_s - lse) * O_s.
 * A part with lse_s = -inf saw no token and has weight 0; if every part is
 * empty the row is out = 0, lse = -inf. NaN inputs propagate.
 *   part_out float [S, R, 512], part_lse float [S, R]
 *   out double [R, 512], lse double [R]
 */
void oracle_combine(int32_t S, int64_t R, const float* part_out, const float* part_lse,
                    double* out, double* lse) {
  for (int64_t r = 0; r < R; ++r) {
    double m = -INFINITY;
    int any_nan = 0;
    for (int32_t s = 0; s < S; ++s) {
      const double v = part_lse[(int64_t)s * R + r];
      if (isnan(v)) any_nan = 1;
      if (v > m) m = v;
    }
    double* o = out + r * D_LATENT;
    if (any_nan) {
      for (int e = 0; e < D_LATENT; ++e) o[e] = NAN;
      lse[r] = NAN;
      continue;
    }
    for (int e = 0; e < D_LATENT; ++e) o[e] = 0.0;
    if (m == -INFINITY) {
      lse[r] = -INFINITY;
      continue;
    }
    double total = 0.0;
    for (int32_t s = 0; s < S; ++s) total += exp((double)part_lse[(int64_t)s * R + r] - m);
    const double L = m + log(total);
    for (int32_t s = 0; s < S; ++s) {
      const double w = exp((double)part_lse[(int64_t)s * R + r] - L);
      if (w == 0.0) continue;
      const float* po = part_out + ((int64_t)s * R + r) * D_LATENT;
      for (int e = 0; e < D_LATENT; ++e) o[e] += w * (double)po[e];
    }
    lse[r] = L;
  }
}

/* ---------------------------------------------------------- split plan */

/*
 * The work partition the GPU library uses (its own rule, stated here from
 * the library's header): let nb_b = ceil(L_b / 64) with L_b clamped as in
 * seq_tokens, pre_b = sum_{b'<b} nb_b', T = pre_B. The T blocks, laid end
 * to end in sequence order, are cut into P parts; part p covers
 * [floor(p T / P), floor((p+1) T / P)). The part holding block x is
 * ceil((x+1) P / T) - 1. A non-empty sequence spans parts first..last
 * (the parts holding its first and its last block); an empty sequence is
 * owned by the part holding block pre_b, or by part P-1 when pre_b == T.
 *   seq_prefix [B+1], part_start [P+1], seq_first_part [B], seq_last_part [B]
 */
int oracle_plan(int32_t B, const int32_t* seqlens, int32_t max_blocks, int32_t P,
                int32_t* seq_prefix, int32_t* part_start, int32_t* seq_first_part,
                int32_t* seq_last_part) {
  if (P < 1 || B < 0) return -1;
  int64_t acc = 0;
  for (int32_t b = 0; b < B; ++b) {
    seq_prefix[b] = (int32_t)acc;
    acc += (seq_tokens(seqlens, b, max_blocks) + BLOCK_TOKENS - 1) / BLOCK_TOKENS;
  }
  seq_prefix[B] = (int32_t)acc;
  const int64_t T = acc;
  for (int32_t p = 0; p <= P; ++p) part_start[p] = (int32_t)((int64_t)p * T / P);
  for (int32_t b = 0; b < B; ++b) {
    const int64_t lo = seq_prefix[b], hi = seq_prefix[b + 1];
    if (hi > lo) {
      seq_first_part[b] = (int32_t)(((lo + 1) * P + T - 1) / T - 1);
      seq_last_part[b] = (int32_t)((hi * P + T - 1) / T - 1);
    } else {
      const int32_t owner = lo < T ? (int32_t)(((lo + 1) * P + T - 1) / T - 1) : P - 1;
      seq_first_part[b] = owner;
      seq_last_part[b] = owner;
    }
  }
  return 0;
}
