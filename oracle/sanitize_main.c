/*
 * Host-side memory and undefined-behaviour check of the oracle (test
 * infrastructure): built with gcc -fsanitize=address,undefined together with
 * mla_oracle.c by tests/test_oracle_sanitized.py, it drives every oracle
 * entry point over small inputs that reach the edge paths (empty and
 * one-token sequences, a tail block, an invalid block id, clamped seqlens, a
 * causal pair, empty and NaN parts in the merge, skipped append rows) for
 * the four cache types and for rows given as doubles. Any out-of-bounds access, use of uninitialised heap,
 * signed overflow or other undefined behaviour aborts the run; the results
 * themselves are checked by the other oracle tests.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#define D_K 576
#define D_L 512
#define D_R 64
#define D_H 128
#define BT 64

int oracle_decode_absorbed(int32_t B, int32_t s_q, int32_t H, const uint16_t* q, int32_t kv_kind,
                           const void* kv, const void* kv_scales, int64_t num_blocks,
                           const int32_t* block_table, int32_t max_blocks, const int32_t* seqlens,
                           double softmax_scale, const int64_t* rows, int64_t n_rows, double* out,
                           double* lse);
int oracle_decode_absorbed_abs(int32_t B, int32_t s_q, int32_t H, const uint16_t* q,
                               int32_t kv_kind, const void* kv, const void* kv_scales,
                               int64_t num_blocks, const int32_t* block_table, int32_t max_blocks,
                               const int32_t* seqlens, double softmax_scale, const int64_t* rows,
                               int64_t n_rows, double* out, double* lse, double* out_abs);
int oracle_decode_decompressed(int32_t B, int32_t s_q, int32_t H, const double* q_nope,
                               const double* q_rope, const double* w_uk, const double* w_uv,
                               const uint16_t* kv, int64_t num_blocks, const int32_t* block_table,
                               int32_t max_blocks, const int32_t* seqlens, double softmax_scale,
                               double* out, double* lse);
void oracle_absorb_query(int64_t rows, int32_t H, const double* q_nope, const double* q_rope,
                         const double* w_uk, double* q_abs);
void oracle_project_output(int64_t rows, int32_t H, const double* o_lat, const double* w_uv,
                           double* o);
void oracle_combine(int32_t S, int64_t R, const float* part_out, const float* part_lse,
                    double* out, double* lse);
int oracle_plan(int32_t B, const int32_t* seqlens, int32_t max_blocks, int32_t P,
                int32_t* seq_prefix, int32_t* part_start, int32_t* seq_first_part,
                int32_t* seq_last_part);
int64_t oracle_cache_append(int32_t B, int32_t s_q, int32_t kind, const uint16_t* rows,
                            const int32_t* block_table, int32_t max_blocks, const int32_t* seqlens,
                            int64_t num_blocks, void* kv, void* scales);
void oracle_quantize_q8_0_row(const float* x, int8_t* q, uint16_t* scales);
void oracle_quantize_fp8_row(const float* x, uint8_t* q, float* scale);
void oracle_quantize_q4h_row(const float* x, uint8_t* q, uint16_t* scales);
void oracle_hadamard32(const double* x, double* y);
void oracle_q4h_dequantize(int64_t rows, const uint8_t* codes, const uint16_t* scales,
                           double* out);

static uint64_t state = 0x9e3779b97f4a7c15ull;
static uint32_t next_u32(void) {   /* xorshift64*: any deterministic filler will do */
  state ^= state >> 12;
  state ^= state << 25;
  state ^= state >> 27;
  return (uint32_t)((state * 0x2545f4914f6cdd1dull) >> 32);
}
static float next_f(void) { return ((float)(next_u32() >> 8) / 16777216.0f - 0.5f) * 4.0f; }
static uint16_t next_bf16(void) {
  const float f = next_f();
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}
static void* xmalloc(size_t n) {
  void* p = malloc(n ? n : 1);
  if (!p) {
    fprintf(stderr, "out of memory\n");
    exit(2);
  }
  return p;
}

int main(void) {
  /* 5 sequences: empty, one token, a tail block, one whose second block id is
   * out of the pool, and one whose seqlen 1000 > 64 * max_blocks is clamped */
  enum { B = 5, S_Q = 2, H = 8, MAXB = 3, NBLK = 8 };
  const int32_t seqlens[B] = {0, 1, 100, 130, 1000};
  int32_t table[B * MAXB] = {0, 1, 2, 3, -1, -1, 4, 5, -1, 6, 99, 7, 2, 3, 4};
  const int64_t rows = (int64_t)B * S_Q * H;
  uint16_t* q = xmalloc(sizeof(uint16_t) * rows * D_K);
  for (int64_t i = 0; i < rows * D_K; ++i) q[i] = next_bf16();
  uint16_t* kv16 = xmalloc(sizeof(uint16_t) * NBLK * BT * D_K);
  for (int64_t i = 0; i < (int64_t)NBLK * BT * D_K; ++i) kv16[i] = next_bf16();
  int8_t* kv8 = xmalloc((size_t)NBLK * BT * D_K);
  uint16_t* sc16 = xmalloc(sizeof(uint16_t) * NBLK * BT * (D_K / 32));
  uint8_t* kvf8 = xmalloc((size_t)NBLK * BT * D_K);
  float* sc32 = xmalloc(sizeof(float) * NBLK * BT);
  uint8_t* kv4 = xmalloc((size_t)NBLK * BT * (D_K / 2));
  uint16_t* sc4 = xmalloc(sizeof(uint16_t) * NBLK * BT * (D_K / 32));
  float row[D_K];
  for (int64_t r = 0; r < (int64_t)NBLK * BT; ++r) {
    for (int e = 0; e < D_K; ++e) row[e] = next_f();
    if (r == 5) memset(row, 0, sizeof(row));    /* an all-zero row: scale 0 */
    oracle_quantize_q8_0_row(row, kv8 + r * D_K, sc16 + r * (D_K / 32));
    oracle_quantize_fp8_row(row, kvf8 + r * D_K, sc32 + r);
    oracle_quantize_q4h_row(row, kv4 + r * (D_K / 2), sc4 + r * (D_K / 32));
  }
  {
    double hx[32], hy[32];
    for (int j = 0; j < 32; ++j) hx[j] = next_f();
    oracle_hadamard32(hx, hy);
  }
  double* out = xmalloc(sizeof(double) * rows * D_L);
  double* lse = xmalloc(sizeof(double) * rows);
  double* oabs = xmalloc(sizeof(double) * rows * D_L);
  double* kvd = xmalloc(sizeof(double) * NBLK * BT * D_K);
  oracle_q4h_dequantize((int64_t)NBLK * BT, kv4, sc4, kvd);
  const void* kvs[5] = {kv16, kv8, kvf8, kv4, kvd};
  const void* scs[5] = {NULL, sc16, sc32, sc4, NULL};
  for (int kind = 0; kind < 5; ++kind) {
    if (oracle_decode_absorbed(B, S_Q, H, q, kind, kvs[kind], scs[kind], NBLK, table, MAXB, seqlens,
                               0.07, NULL, 0, out, lse) != 0)
      return 3;
    const int64_t pick[4] = {0, 17, rows - 1, 40};
    if (oracle_decode_absorbed_abs(B, S_Q, H, q, kind, kvs[kind], scs[kind], NBLK, table, MAXB,
                                   seqlens, 0.07, pick, 4, out, lse, oabs) != 0)
      return 4;
  }
  /* a row id out of range is refused */
  const int64_t bad_row = rows;
  if (oracle_decode_absorbed(B, S_Q, H, q, 0, kv16, NULL, NBLK, table, MAXB, seqlens, 0.07,
                             &bad_row, 1, out, lse) != -1)
    return 5;

  /* decompressed definition, absorption and projection */
  double* qn = xmalloc(sizeof(double) * rows * D_H);
  double* qr = xmalloc(sizeof(double) * rows * D_R);
  double* wk = xmalloc(sizeof(double) * H * D_H * D_L);
  double* wv = xmalloc(sizeof(double) * H * D_H * D_L);
  double* qa = xmalloc(sizeof(double) * rows * D_K);
  double* o = xmalloc(sizeof(double) * rows * D_H);
  for (int64_t i = 0; i < rows * D_H; ++i) qn[i] = next_f();
  for (int64_t i = 0; i < rows * D_R; ++i) qr[i] = next_f();
  for (int64_t i = 0; i < (int64_t)H * D_H * D_L; ++i) wk[i] = next_f() * 0.05;
  for (int64_t i = 0; i < (int64_t)H * D_H * D_L; ++i) wv[i] = next_f() * 0.05;
  oracle_decode_decompressed(B, S_Q, H, qn, qr, wk, wv, kv16, NBLK, table, MAXB, seqlens, 0.07, o,
                             lse);
  oracle_absorb_query(rows, H, qn, qr, wk, qa);
  double* ol = xmalloc(sizeof(double) * rows * D_L);
  for (int64_t i = 0; i < rows * D_L; ++i) ol[i] = next_f();
  oracle_project_output(rows, H, ol, wv, o);

  /* merge: three parts, one empty (-inf), one row poisoned (NaN) */
  enum { S = 3, R = 7 };
  float* po = xmalloc(sizeof(float) * S * R * D_L);
  float pl[S * R];
  for (int i = 0; i < S * R * D_L; ++i) po[i] = next_f();
  for (int i = 0; i < S * R; ++i) pl[i] = next_f();
  for (int r = 0; r < R; ++r) pl[1 * R + r] = -INFINITY;
  pl[2 * R + 4] = NAN;
  oracle_combine(S, R, po, pl, out, lse);

  /* plan for several part counts, including more parts than blocks */
  int32_t pre[B + 1], ps[65], first[B], last[B];
  const int32_t parts[4] = {1, 3, 7, 64};
  for (int i = 0; i < 4; ++i)
    if (oracle_plan(B, seqlens, MAXB, parts[i], pre, ps, first, last) != 0) return 6;

  /* append into each cache type; rows outside the table or in the bad block
   * are skipped */
  uint16_t* new_rows = xmalloc(sizeof(uint16_t) * B * S_Q * D_K);
  for (int i = 0; i < B * S_Q * D_K; ++i) new_rows[i] = next_bf16();
  void* kv_app[4] = {kv16, kv8, kvf8, kv4};
  void* sc_app[4] = {NULL, sc16, sc32, sc4};
  for (int kind = 0; kind < 4; ++kind)
    (void)oracle_cache_append(B, S_Q, kind, new_rows, table, MAXB, seqlens, NBLK, kv_app[kind],
                              sc_app[kind]);

  free(q); free(kv16); free(kv8); free(sc16); free(kvf8); free(sc32); free(kv4); free(sc4);
  free(kvd);
  free(out); free(lse);
  free(oabs); free(qn); free(qr); free(wk); free(wv); free(qa); free(o); free(ol); free(po);
  free(new_rows);
  printf("oracle sanitizer run: ok\n");
  return 0;
}
