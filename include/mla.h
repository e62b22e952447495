/*
 * libmla -- Multi-Head Latent Attention decode over a paged latent cache,
 * for AMD Instinct MI355X (gfx950).
 *
 * What is computed. MLA caches one compressed latent vector c_KV per token
 * (512 values here) and recovers keys and values through up-projections
 * k = W_UK c, v = W_UV c ("MLA: Multi-Head Latent Attention -- DeepSeek-AI
 * Explained", section Method, architecture equations). Folding W_UK into the
 * query and W_UV into the output projection (the weight-absorbing trick:
 * nnets.ru article on MLA and FlashAttention, section on the essence of MLA;
 * snowgate.dev forum thread 35, last reply) lets every head attend directly
 * to the cached rows, and the RoPE part of the key travels as a separate
 * 64-wide slice shared by all heads (thread 35, replies on the 512 + 64 row).
 * So each cached token row is [c_KV (512) | k_rope (64)] = 576 values, each
 * query row is the absorbed query [W_UK^T q_nope ; q_rope] (576 values), and
 * for every query row
 *
 *     s_t  = softmax_scale * <q, row_t>           over the 576 columns
 *     out  = sum_t softmax(s)_t * row_t[0:512]    (the latent is V)
 *     lse  = ln sum_t exp(s_t)
 *
 * over the tokens the row may see. The result stays in the 512-wide latent
 * space; applying W_UV and W_O is the caller's business. No per-head K or V
 * is ever built. This is exact softmax attention evaluated FlashAttention-
 * style (FlashMLA page of the ik_llama.cpp docs, "What is MLA?"); the
 * optional q8_0 cache follows "KV cache with MLA" on the same page, and so
 * does the q4_0 cache whose keys are Hadamard-transformed before
 * quantisation (there the option recommended below 6-bit caches).
 *
 * Layouts (all row-major and contiguous):
 *   q            bf16  [B, s_q, H, 576]        query row r = i*H + h of sequence b
 *   kv_cache     bf16  [num_blocks, 64, 576]   (MLA_KV_BF16)
 *                int8  [num_blocks, 64, 576]   (MLA_KV_Q8_0) with
 *   kv_scales    fp16  [num_blocks, 64, 18]    scale g covers columns 32g .. 32g+31;
 *                                              a cached value is scale * int8
 *                uint8 [num_blocks, 64, 576]   (MLA_KV_FP8: OCP e4m3, 1-4-3, bias 7) with
 *   kv_scales    fp32  [num_blocks, 64]        one scale per token; a cached value
 *                                              is scale * e4m3 (576 + 4 bytes a token)
 *                uint8 [num_blocks, 64, 288]   (MLA_KV_Q4_0H: 4-bit codes, two per
 *                                              byte, code j of block g in byte
 *                                              16 g + j / 2, low nibble for even j) with
 *   kv_scales    fp16  [num_blocks, 64, 18]    block g = columns 32g .. 32g+31 holds
 *                                              y = d_g * (code - 8) and stands for the
 *                                              cached values R y, R = H / sqrt(32), H
 *                                              the 32-point Sylvester-Hadamard matrix
 *                                              (H[m][j] = (-1)^popcount(m & j)); R is
 *                                              its own inverse (288 + 36 bytes a token)
 *   block_table  int32 [B, max_blocks_per_seq] token t of sequence b is row t % 64
 *                                              of block block_table[b][t / 64]
 *   seqlens      int32 [B]                     cached tokens of sequence b,
 *                                              including its s_q new tokens
 *   out          bf16  [B, s_q, H, 512]
 *   lse          fp32  [B, s_q, H]             natural log
 *
 * Visibility: query i (0 <= i < s_q) of sequence b sees tokens
 * 0 .. seqlens[b] - s_q + i (causal among the new tokens). A row that sees no
 * token gets out = 0 and lse = -inf. seqlens are clamped to
 * [0, 64 * max_blocks_per_seq]. If any block id a sequence uses lies outside
 * [0, num_blocks), every out and lse value of that sequence is NaN and no
 * out-of-range block is read.
 *
 * Pointers: every array argument is a device pointer unless marked host. The
 * caller owns all memory; the library keeps no pointer after a call returns
 * and allocates nothing. Calls only enqueue work on `stream` (no host
 * synchronisation); inputs must stay alive until the stream has passed them.
 * Errors found on the host are returned before anything is enqueued, and
 * nothing is written then. Results are deterministic for fixed inputs and a
 * fixed problem descriptor (no floating-point atomics).
 *
 * Alignment: q, kv_cache, kv_scales, out and the workspace must be 16-byte
 * aligned; lse, block_table and seqlens 4-byte.
 */
#ifndef LIBMLA_MLA_H
#define LIBMLA_MLA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_D_LATENT 512
#define MLA_D_ROPE 64
#define MLA_D_K 576
#define MLA_D_HEAD 128       /* per-head no-RoPE query width and value width */
#define MLA_BLOCK_TOKENS 64
#define MLA_Q8_GROUP 32
#define MLA_MAX_BATCH 2048   /* sequences per call */
#define MLA_MAX_ROWS 4096    /* s_q * H */
/* Device workspace held by mla_decode_noalloc (per device, for the life of
 * the process): enough for every automatic split plan on a 256-CU MI355X
 * (at most 2 * 256 * 128 query rows of bf16 partials, 67.4 MB). */
#define MLA_NOALLOC_SCRATCH_BYTES ((size_t)72 << 20)

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = 1,        /* null pointer, bad size, misaligned pointer */
  MLA_ERR_UNSUPPORTED = 2,        /* outside the supported limits */
  MLA_ERR_WORKSPACE_TOO_SMALL = 3,
  MLA_ERR_HIP = 4                 /* a HIP runtime call or launch failed */
} mla_status;

typedef enum { MLA_KV_BF16 = 0, MLA_KV_Q8_0 = 1, MLA_KV_FP8 = 2, MLA_KV_Q4_0H = 3 } mla_kv_dtype;

/* Problem descriptor (host struct, read during a call only). */
typedef struct {
  int32_t batch;              /* B, 0 .. MLA_MAX_BATCH */
  int32_t seqlen_q;           /* s_q >= 1: new query tokens per sequence */
  int32_t num_heads;          /* H >= 1, s_q * H <= MLA_MAX_ROWS */
  int32_t max_blocks_per_seq; /* block_table row stride, >= 1 */
  int64_t num_blocks;         /* blocks in the cache pool, >= 0 */
  int32_t max_seqlen;         /* host-known bound on seqlens used to size the work
                                 split; 0 means 64 * max_blocks_per_seq. Results do
                                 not depend on it. */
  int32_t kv_dtype;           /* mla_kv_dtype */
  int32_t num_parts;          /* 0: automatic; else P >= 1 KV partitions (see mla_plan) */
  int32_t m_tile;             /* 0: automatic; else 16, 32, 64 or 128 query rows
                                 per workgroup (16: bf16 cache only; fp8 cache:
                                 128 only). Automatic picks the smallest tile
                                 that holds seqlen_q * num_heads rows (16 only
                                 for bf16), else 128; always 128 for fp8. */
} mla_problem;

/* Bytes of device workspace mla_decode needs for *p (written to *bytes, host).
 * The size depends only on the descriptor and the device's compute-unit count. */
mla_status mla_workspace_size(const mla_problem* p, size_t* bytes);

/* Number of KV partitions P that mla_decode uses for *p (written to *num_parts, host). */
mla_status mla_num_parts(const mla_problem* p, int32_t* num_parts);

/*
 * Decode one step: out and lse for every query row of every sequence, as
 * defined at the top of this file. Uses split-KV partitions when that fills
 * the GPU better, with a log-sum-exp merge of the partial results (the same
 * merge as mla_combine; inside the workspace a partial result is held as
 * bf16 of the part's normalised output, plus its fp32 lse). workspace: device buffer of at least
 * mla_workspace_size bytes (may be NULL when that size is 0); its contents on
 * entry do not matter and are overwritten.
 */
mla_status mla_decode(const mla_problem* p, const void* q, const void* kv_cache,
                      const void* kv_scales, const int32_t* block_table,
                      const int32_t* seqlens, float softmax_scale, void* out, float* lse,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * mla_decode without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation). The workspace is a library-owned device array of
 * MLA_NOALLOC_SCRATCH_BYTES per device, created with the library's code
 * object and held until the process ends; its address is looked up once per
 * device on the first call made with that device current. The call itself
 * makes no allocation of any kind. Arguments, results and errors are those of
 * mla_decode (same kernels, same plan, bit-identical results), plus
 * MLA_ERR_UNSUPPORTED when the problem's workspace (mla_workspace_size) would
 * exceed MLA_NOALLOC_SCRATCH_BYTES; nothing is enqueued then. Every call on a
 * device shares that device's array, which keeps the last call's contents:
 * calls whose executions overlap on one device (several streams, several host
 * threads) race and give undefined results; serialise them.
 */
mla_status mla_decode_noalloc(const mla_problem* p, const void* q, const void* kv_cache,
                              const void* kv_scales, const int32_t* block_table,
                              const int32_t* seqlens, float softmax_scale, void* out,
                              float* lse, hipStream_t stream);

/*
 * Log-sum-exp merge of num_splits partial results of the same rows, each
 * computed over a disjoint set of tokens:
 *     lse[r] = ln sum_s exp(partial_lse[s][r])
 *     out[r] = sum_s exp(partial_lse[s][r] - lse[r]) * partial_out[s][r]
 * A part with lse = -inf saw no token and has weight 0; rows whose parts are
 * all empty get out = 0, lse = -inf; NaN in any part gives NaN.
 *   partial_out fp32 [num_splits, rows, 512], partial_lse fp32 [num_splits, rows]
 *   out bf16 [rows, 512], lse fp32 [rows]
 * num_splits >= 1, rows >= 0. This is the merge that makes split-KV decoding
 * exact (split the tokens, attend to each part, merge), which is how one
 * long sequence can be spread over many compute units or devices.
 */
mla_status mla_combine(int32_t num_splits, int64_t rows, const float* partial_out,
                       const float* partial_lse, void* out, float* lse, hipStream_t stream);

/*
 * The work partition mla_decode uses, computed on the device from seqlens.
 * With nb_b = ceil(L_b / 64) (L_b clamped as above), pre_b = sum_{b'<b} nb_b'
 * and T = pre_B, the T cache blocks laid end to end in sequence order are cut
 * into P = mla_num_parts(p) parts; part p covers blocks
 * [floor(p*T/P), floor((p+1)*T/P)), and block x lies in part
 * ceil((x+1)*P/T) - 1. A non-empty sequence spans the parts holding its first
 * and its last block; an empty one is owned by the part holding block pre_b
 * (part P-1 if pre_b == T). Each part is processed by one workgroup per
 * query-row tile.
 * Writes int32 to plan_out (device, capacity plan_capacity int32 values,
 * at least 3*B + P + 2): seq_prefix [B+1], part_start [P+1],
 * seq_first_part [B], seq_last_part [B], concatenated in that order.
 */
mla_status mla_plan(const mla_problem* p, const int32_t* seqlens, int32_t* plan_out,
                    int64_t plan_capacity, hipStream_t stream);

/*
 * The steps either side of mla_decode (a decoder layer's MLA attention in
 * absorbed form). MLA rebuilds per-head keys and values from the cached
 * latent as k = W_UK c and v = W_UV c ("MLA: Multi-Head Latent Attention --
 * DeepSeek-AI Explained", section Method); absorbing W_UK into the query and
 * W_UV into the output (nnets.ru article, section on the essence of MLA;
 * snowgate.dev forum thread 35, last reply) turns them into these two
 * per-head products. Rows are query rows r = (b * s_q + i) * H + h, as in
 * mla_decode; bf16 in and out, fp32 accumulation on the matrix cores.
 * Deterministic; errors are returned before anything is enqueued.
 */

/* q_abs[r] = [ W_UK[h]^T q_nope[r] ; q_rope[r] ]: the absorbed query mla_decode takes.
 *   q_nope bf16 [rows, 128], q_rope bf16 [rows, 64] (already rotated)
 *   w_uk_t bf16 [H, 512, 128]: W_UK[h] transposed, i.e. w_uk_t[h][d][j] = W_UK[h][j][d]
 *          where the per-head key is k_j = sum_d W_UK[h][j][d] c_d
 *   q_abs  bf16 [rows, 576]
 * rows a multiple of num_heads; all arrays 16-byte aligned. */
mla_status mla_absorb_query(int64_t rows, int32_t num_heads, const void* q_nope,
                            const void* q_rope, const void* w_uk_t, void* q_abs,
                            hipStream_t stream);

/* o[r] = W_UV[h] o_lat[r]: the per-head attention output from mla_decode's
 * latent-space output.
 *   o_lat bf16 [rows, 512], w_uv bf16 [H, 128, 512] (v_j = sum_d W_UV[h][j][d] c_d),
 *   o     bf16 [rows, 128]
 * rows a multiple of num_heads; all arrays 16-byte aligned. */
mla_status mla_project_output(int64_t rows, int32_t num_heads, const void* o_lat,
                              const void* w_uv, void* o, hipStream_t stream);

/* Append the s_q new tokens of a decode step to the paged cache, before
 * mla_decode reads it: row i of sequence b (rows bf16 [B, s_q, 576], the new
 * [c_KV | k_rope] with k_rope already rotated) is token t = seqlens[b] - s_q + i
 * and goes to row t % 64 of block block_table[b][t / 64]. Rows whose position
 * falls outside [0, 64 * max_blocks_per_seq) or whose block id lies outside
 * [0, num_blocks) are skipped.
 *   MLA_KV_BF16: kv_cache bf16 [num_blocks, 64, 576], the row copied as is;
 *   MLA_KV_Q8_0: kv_cache int8 [num_blocks, 64, 576] + kv_scales fp16
 *     [num_blocks, 64, 18], written by the q8_0 rule (FlashMLA page of the
 *     ik_llama.cpp docs, "KV cache with MLA"): per group g of 32 columns,
 *     d = max |x| / 127 in fp32, scale = fp16(d) rounded to nearest even,
 *     code = x / d rounded half away from zero, clamped to [-127, 127]
 *     (max |x| = 0 gives scale 0 and codes 0);
 *   MLA_KV_FP8: kv_cache uint8 [num_blocks, 64, 576] + kv_scales fp32 [num_blocks, 64]:
 *     one scale per token, d = max |x| / 448 (fp32, stored as is), code = OCP E4M3
 *     of x / d, nearest even, saturated to +-448 (the forum's fp8 KV cache,
 *     snowgate.dev thread 35); max |x| = 0 gives scale 0 and codes 0;
 *   MLA_KV_Q4_0H: kv_cache uint8 [num_blocks, 64, 288] + kv_scales fp16
 *     [num_blocks, 64, 18]: each block g of 32 columns is rotated by the
 *     Hadamard matrix before it is quantised (FlashMLA page, "KV cache with
 *     MLA", the K-cache Hadamard option for low-bit caches), in fp32: the fast
 *     transform (for strides 1, 2, 4, 8, 16 every pair (a, b) -> (a + b, a - b)),
 *     then each value times fp32(1 / sqrt(32)); then q4_0: m = the first value
 *     of largest magnitude, d = m / -8, code = min(15, floor(y / d + 8.5)) (all
 *     codes 8 when d = 0), scale = fp16(d) to nearest even.
 * rows must be finite.
 * rows and kv_cache 16-byte aligned, the other arrays 4-byte. Two new rows
 * aimed at the same slot race. */
mla_status mla_cache_append(int32_t batch, int32_t seqlen_q, const void* rows,
                            const int32_t* block_table, int32_t max_blocks_per_seq,
                            const int32_t* seqlens, int64_t num_blocks, int32_t kv_dtype,
                            void* kv_cache, void* kv_scales, hipStream_t stream);

/* Static description of a status code. */
const char* mla_status_str(mla_status s);

/* Detail of the last error returned on the calling thread ("" if none). */
const char* mla_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBMLA_MLA_H */
