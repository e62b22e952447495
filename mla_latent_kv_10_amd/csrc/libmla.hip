// libmla: MLA decode in weight-absorbed form over a paged latent cache, for
// gfx950 (MI355X). The operation and the C ABI are defined in include/mla.h.
//
// Design in brief (CDNA4):
//  * One workgroup = 4 waves on one CU (8 for the 64-row quantised tile),
//    processing one KV partition of the cache for a tile of query rows:
//    16 rows (mla_decode_narrow_kernel), 32 or 64 (mla_decode_rows_kernel),
//    128 (mla_decode_pipe_kernel) for a bf16 cache; 128 for an fp8 cache
//    (the pipe kernel reading E4M3 codes); 32 or 64 (mla_decode_kernel) and
//    128 (mla_decode_q8w_kernel) for a q8_0 cache and for a q4_0 cache stored
//    in Hadamard rotation.
//  * The cache streams through LDS in 32-token tiles (half a 64-token block,
//    36 KiB in bf16), fetched with global_load_lds_dwordx4 (direct to LDS, no
//    VGPRs) into a 3- or 4-stage ring, so two or three tiles are in flight
//    while one is consumed. In the 128- and 16-row kernels each copy
//    instruction reads eight whole 128-byte lines (row-group tile layouts),
//    which allows the non-temporal cache policy for tiles read only once.
//  * Scores are computed transposed, S^T = K q~^T, with tokens on the M side
//    and heads on the N side of the MFMA: each lane's accumulator then holds
//    tokens of one head, which is the B-operand layout of the value product
//    O^T += V^T P^T. V^T operands come from the same LDS tile through
//    ds_read_b64_tr_b16 (transposing reads), since V is the latent itself.
//  * Online softmax in the log2 domain (exp2 on v_exp_f32), fp32 accumulators,
//    with a reference maximum that moves rarely (so the accumulators are
//    rarely rescaled).
//  * Split-KV: the blocks of all sequences, laid end to end, are cut into P
//    equal parts (the plan, recomputed from seqlens inside every kernel, so
//    the host never synchronises). A sequence that spans parts leaves bf16
//    partials (normalised O and lse) and a second kernel merges them with a
//    log-sum-exp combine.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <stdarg.h>
#include <stdlib.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <type_traits>
#include <utility>
#include <string>

#include "mla.h"

namespace {

constexpr int kDL = MLA_D_LATENT;           // 512: latent width = V width
constexpr int kDK = MLA_D_K;                // 576: K row width
constexpr int kBT = MLA_BLOCK_TOKENS;       // 64 tokens per cache block
constexpr int kTile = 32;                   // tokens per LDS tile
constexpr int kRowBytes = kDK * 2;          // 1152 bytes per bf16 row
constexpr int kTileBytes = kTile * kRowBytes;   // 36864
constexpr int kThreads = 256;
constexpr int kStages = 3;
constexpr int kMaxBatch = MLA_MAX_BATCH;
// q8_0 tiles: 32 rows x 576 int8 plus 32 rows x 18 fp16 scales
constexpr int kQ8RowBytes = kDK;            // 576
constexpr int kQ8ScaleRowBytes = 36;
constexpr int kQ8TileBytes = kTile * kQ8RowBytes;               // 18432
constexpr int kQ8ScaleTileBytes = kTile * kQ8ScaleRowBytes;     // 1152
constexpr int kQ8StageBytes = kQ8TileBytes + 2048;              // int8 + scales, padded
// q4_0 tiles in Hadamard rotation: 32 rows x 288 code bytes plus the same
// 32 x 18 fp16 scales; code block g of token t is 16-byte unit 32 g + t
constexpr int kQ4RowBytes = kDK / 2;        // 288
constexpr int kQ4TileBytes = kTile * kQ4RowBytes;               // 9216
constexpr int kQ4StageBytes = kQ4TileBytes + 2048;              // codes + scales, padded
constexpr float kInvSqrt32 = 0.17677669529663688f;               // 1 / sqrt(32)
// fp8 (e4m3) tiles: 32 rows x 576 bytes plus 32 fp32 per-token scales
constexpr int kFp8TileBytes = kTile * kDK;                      // 18432
constexpr int kFp8StageBytes = kFp8TileBytes + 1024;            // fp8 + scales, padded

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef short i16x4 __attribute__((__vector_size__(4 * sizeof(short))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));
typedef uint32_t u32x2 __attribute__((__vector_size__(2 * sizeof(uint32_t))));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x8 __attribute__((__vector_size__(8 * sizeof(uint32_t))));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Eight OCP E4M3 codes (byte i = element i) to bf16, exactly: every finite
// E4M3 value, subnormals included, is a bf16 value.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(u32x2 w) {
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, false));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, true));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, false));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, true));
  return __builtin_bit_cast(bf16x8, r);
}

#define LDS_AS __attribute__((address_space(3)))
// Read-only for the whole kernel: loads through this address space with a
// uniform address become scalar loads (s_load, counted by lgkmcnt) instead of
// vector loads, so they never wait behind the LDS-DMA loads in flight.
#define CONST_AS __attribute__((address_space(4)))

struct DecodeParams {
  const uint16_t* q;
  const uint8_t* kv;
  const uint8_t* kv_scales;
  const int32_t* block_table;
  const int32_t* seqlens;
  uint16_t* out;
  float* lse;
  int32_t* ws_prefix;   // [B+1] block prefix, written by workgroup 0
  float* part_lse;      // [2P, M]
  uint16_t* part_o;     // [2P, M, 512] bf16: partial results of split sequences
  int64_t num_blocks;
  int B, s_q, H, M, max_blocks, P, m_tiles;
  float scale_log2;     // softmax_scale * log2(e)
  float scale_mag_log2; // |softmax_scale| * log2(e)
  uint32_t q_sign2;     // 0x80008000 when softmax_scale < 0: the query is negated
                        // instead, so the scale applied in the kernel is >= 0
};

// ------------------------------------------------------------------ helpers

__device__ __forceinline__ int clamp_len(int L, int max_blocks) {
  return L < 0 ? 0 : (L > max_blocks * kBT ? max_blocks * kBT : L);
}

__device__ __forceinline__ int nblocks_of(int L, int max_blocks) {
  return (clamp_len(L, max_blocks) + kBT - 1) / kBT;
}

// Part holding flattened block x (T > 0): ceil((x+1) P / T) - 1.
__device__ __forceinline__ int part_of(int x, int P, int T) {
  return (int)((((int64_t)x + 1) * P + T - 1) / T - 1);
}

__device__ __forceinline__ int part_start(int p, int P, int T) {
  return (int)((int64_t)p * T / P);
}

// Wait until at most N vector-memory operations of this wave are pending.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for LDS traffic only. __syncthreads() would also wait for
// every outstanding global load (vmcnt(0)), including the LDS-DMA prefetch of
// later tiles; callers wait for exactly the loads they need first.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
  return (uint32_t)(uintptr_t)(const LDS_AS void*)p;
}

__device__ __forceinline__ bf16x8 lds_read_b128(const LDS_AS uint8_t* p) {
  return *reinterpret_cast<const LDS_AS bf16x8*>(p);
}

// V^T operand of the value product for one lane: two transposing 64-bit
// reads (tokens +0..3 and +8..11 of the fragment). In each 16-lane group,
// lane 4s+q points at columns 4q..4q+3 of token s, and lane i receives
// column i of tokens s = 0..3 (ds_read_b64_tr_b16).
__device__ __forceinline__ bf16x8 vt_fragment(const LDS_AS uint8_t* p0, const LDS_AS uint8_t* p1) {
  i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(p0));
  i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(p1));
  typedef short i16x8 __attribute__((__vector_size__(8 * sizeof(short))));
  i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// The same operand from an fp8 (E4M3) tile, as codes: one transposing
// 64-bit read (in each 16-lane group, lane 2s+h points at columns 8h..8h+7
// of token s and lane i receives column i of tokens s = 0..7).
__device__ __forceinline__ u32x2 vt_codes8(const LDS_AS uint8_t* p) {
  const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS i32x2*)(p));
  return u32x2{(uint32_t)v[0], (uint32_t)v[1]};
}

// LDS tile layout of the 32/64-row and q8_0 kernels (bf16, 32 tokens x 576
// columns = 36 KiB): chunk-major in 16-byte units (8 columns of one token). Unit 32c + (t ^ 4(c & 3)) holds
// columns 8c..8c+7 of token t. Reading one chunk row for 32 tokens (the
// score operand) covers 512 contiguous bytes; the XOR spreads the four
// chunks a 32-lane half touches in a transposing read (the value operand)
// over the four 64-byte quarters of the bank window.
__device__ __forceinline__ int tile_unit(int t, int c) { return 32 * c + (t ^ (4 * (c & 3))); }

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Block-wide exclusive prefix of cache blocks per sequence: s_pre[0..B].
// Every thread of the workgroup (NT threads) must call it.
// x shifted by n lanes up within each row of 16 lanes, 0 below: one DPP move
template <int N>
__device__ __forceinline__ int row_shr(int x) {
  return __builtin_amdgcn_update_dpp(0, x, 0x110 + N, 0xf, 0xf, true);
}

// Block prefix of the batch: s_pre[b] = blocks of sequences 0..b-1 (B + 1
// entries). Thread t takes sequences t*per .. t*per + per - 1 and keeps their
// block counts in registers; the scan is in-wave (DPP within rows of 16
// lanes, then the row totals by readlane) and across the waves through
// s_wsum[0..3]. Also sets s_wsum[8] = INT_MAX, s_wsum[9] = -1 for part_range.
template <int NT>
__device__ void plan_prefix(const int32_t* __restrict__ seqlens, int B, int max_blocks,
                            int* s_pre, int* s_wsum) {
  constexpr int PER = (kMaxBatch + NT - 1) / NT;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int per = (B + NT - 1) / NT;
  const int lo = min(B, t * per);
  int nb[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k)   // all loads first (per is uniform)
    if (k < per) nb[k] = seqlens[min(lo + k, max(B - 1, 0))];
  int local = 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    nb[k] = k < per && lo + k < B ? nblocks_of(nb[k], max_blocks) : 0;
    local += nb[k];
  }
  int x = local;
  x += row_shr<1>(x);
  x += row_shr<2>(x);
  x += row_shr<4>(x);
  x += row_shr<8>(x);
  const int r0 = __builtin_amdgcn_readlane(x, 15), r1 = __builtin_amdgcn_readlane(x, 31),
            r2 = __builtin_amdgcn_readlane(x, 47);
  const int row = lane >> 4;
  x += (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);   // inclusive
  if (lane == 63) s_wsum[w] = x;
  if (t == 0) {
    s_wsum[8] = 0x7fffffff;
    s_wsum[9] = -1;
  }
  __syncthreads();
  int base = 0;
  for (int i = 0; i < w; ++i) base += s_wsum[i];
  int run = base + x - local;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    if (k < per && lo + k < B) s_pre[lo + k] = run;
    run += nb[k];
  }
  if (t == NT - 1) s_pre[B] = base + x;
  __syncthreads();
}

// The sequences of part `part` (block range [p_lo, p_hi) of the T blocks)
// form a contiguous range [b_first, b_last], empty when b_first > b_last: a
// sequence with blocks belongs to every part whose range meets its own, one
// without blocks to the part that holds its position (the last part when
// the position is T). Uses s_misc[8..9] as plan_prefix left them.
template <int NT>
__device__ void part_range(const int* s_pre, int B, int T, bool last_part, int p_lo, int p_hi,
                           int* s_misc, int& b_first, int& b_last) {
  for (int b = threadIdx.x; b < B; b += NT) {
    const int lo = s_pre[b], hi2 = s_pre[b + 1];
    const bool mine = hi2 > lo ? lo < p_hi && hi2 > p_lo
                               : (lo < T ? lo >= p_lo && lo < p_hi : last_part);
    if (mine) {
      atomicMin(&s_misc[8], b);
      atomicMax(&s_misc[9], b);
    }
  }
  __syncthreads();
  b_first = uniform(s_misc[8]);
  b_last = uniform(s_misc[9]);
}

// ------------------------------------------------------------ decode kernel

// Rescale threshold of the online softmax (log2 units). The reference
// maximum used for the exponentials only moves when a tile's scores exceed
// it by more than this, and when it moves it is set kRefHeadroom above the
// new row maximum, so a later score has to exceed that maximum by 96 before
// the output accumulators are rescaled again: in practice only a segment's
// first tile sets it, even with heavy-tailed scores. The probabilities stay
// below 2^48: bf16 keeps the fp32 exponent range and rounds relatively, and
// the fp32 sums over at most 2^21 tokens stay finite for cache values below
// 5e17. A score 78 or more below the row maximum may underflow to zero; its
// weight relative to the maximum's is then below 2^-78, far under the bf16
// rounding of the probabilities. The result is the same softmax; only the
// reference point changes.
constexpr float kRescaleThreshold = 48.0f;
constexpr float kRefHeadroom = 48.0f;

// 16 bytes per lane from global memory straight into LDS
// (global_load_lds_dwordx4, M0 = LDS base), from an SGPR base and a per-lane
// 32-bit offset (no per-tile address arithmetic); lane l's 16 bytes land at
// lds_addr + 16 l. Issued as inline asm so that the compiler's wait-count
// pass, which cannot tell which ring stage a DMA targets, does not serialise
// every later LDS read behind it; ordering comes from the explicit vmcnt
// waits and LDS barriers. There is no VGPR destination; the offset VGPR is
// read at issue.
__device__ __forceinline__ void dma16_sbase(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds_addr)
               : "memory", "m0");
}

// The same copy with the non-temporal cache policy: the line is not kept in
// L2 for reuse. Only for copies that read whole 128-byte lines each (a line
// read in pieces by several instructions would be fetched once per piece).
__device__ __forceinline__ void dma16_sbase_nt(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt"
               :
               : "v"(voff), "s"(sbase), "s"(lds_addr)
               : "memory", "m0");
}

// f(std::integral_constant<int, I>) for I = 0 .. N-1, fully unrolled.
template <typename F, int... I>
__device__ __forceinline__ void unroll_seq(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void unroll(F&& f) {
  unroll_seq(f, std::make_integer_sequence<int, N>{});
}

// As dma16_sbase with constant offsets added to the lane offset (VADD) and
// to the LDS address (MADD) inside the asm, so that a run of copies shares
// two base registers instead of one hoisted (and spilled) value per copy.
template <int VADD, int MADD>
__device__ __forceinline__ void dma16_sbase_off(const void* sbase, uint32_t voff, uint32_t lds_base) {
  uint32_t t;
  asm volatile("v_add_u32 %0, %5, %1\n\ts_add_u32 m0, %3, %4\n\tglobal_load_lds_dwordx4 %0, %2"
               : "=&v"(t)
               : "v"(voff), "s"(sbase), "s"(lds_base), "n"(MADD), "n"(VADD)
               : "memory", "m0");
}

// Two floats to a bf16 pair (round to nearest even), lo in bits 0..15: one
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  typedef float f32x2v __attribute__((ext_vector_type(2)));
  const f32x2v f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2v));
}

// x - h, for h the bf16 pair holding bf16(x) in its low or high half: one
// v_dot2c_f32_bf16, h times sel plus x, with sel the bf16 pair (-1, 0)
// (bits 0x0000BF80) or (0, -1) (0xBF800000) held in a register (see
// DotSel). The products are exact and so is the difference (h is x
// rounded), so the result is exact whatever the order of the additions.
__device__ __forceinline__ float lo_part(uint32_t h, float x, uint32_t sel) {
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, h), __builtin_bit_cast(bf16x2v, sel),
                                         x, false);
}
// The two selectors of lo_part in VGPRs. Left to the compiler, 0x0000BF80
// becomes the inline constant -1.0, which the hardware reads as the 32-bit
// pattern 0xBF800000, i.e. the other half (measured).
struct DotSel {
  uint32_t lo = 0x0000BF80u, hi = 0xBF800000u;
  __device__ DotSel() { asm volatile("" : "+v"(lo), "+v"(hi)); }
};

// Decode kernel with the work of each 32-row group split over CG waves (the
// q8_0 cache and the q4_0 cache in Hadamard rotation: HG = 1 or 2 row groups,
// CG = 4). The 576-column score
// contraction is split by columns (partial scores summed through LDS) and the
// 512-wide value product by output columns. q8_0: the scores are exact (the
// int8 values are exact in bf16; each 32-column group's partial sum is scaled
// by its fp16 scale in fp32), and the value product reads an LDS tile of
// bf16(scale * int8) written once per tile by all threads.
// Q4 (with Q8): the cache holds, per 32-column block of a row, the q4_0 codes
// of the row's block rotated by R = H / sqrt(32) (H the 32-point
// Sylvester-Hadamard matrix, R its own inverse), so a cached block is
// x = R y = (d / sqrt(32)) H (c - 8). Once per tile all waves form
// n = H (c - 8) for every block of every token on the matrix core (H times
// the tile's codes: integers of magnitude <= 256, exact in bf16 and in the
// fp32 accumulators) into an LDS tile of bf16 n that the score steps read
// in place of the int8 values, the per-group scale being d; 1 / sqrt(32) is
// folded into the softmax scale by the host. The value tile is
// bf16(d / sqrt(32) * n).
template <int HG, int CG, bool Q8, bool Q4 = false>
__global__ __launch_bounds__(64 * HG * CG, 1) void mla_decode_kernel(DecodeParams a) {
  constexpr int NW = HG * CG;             // waves per workgroup
  constexpr int NT = 64 * NW;             // threads
  constexpr int MT = 32 * HG;             // query rows per workgroup
  constexpr int KS = 36 / CG;             // score k-steps (16 columns) per wave
  constexpr int NCT = 16 / CG;            // 32-column output tiles per wave
  constexpr int SL = 16 / CG;             // score registers of this wave's slice
  constexpr int REC = SL / 2 + 2 <= 4 ? 4 : 8;   // dwords per lane in a slice record
  // 1 KiB LDS-DMA loads per tile: code loads, then two of scales (quantised)
  constexpr int CODE_LOADS = Q4 ? 9 : (Q8 ? 18 : 36);
  constexpr int TILE_LOADS = Q8 ? CODE_LOADS + 2 : 36;
  constexpr int STAGE_BYTES = Q4 ? kQ4StageBytes : (Q8 ? kQ8StageBytes : kTileBytes);
  constexpr int SCALE_OFF = Q4 ? kQ4TileBytes : kQ8TileBytes;   // scales in a stage
  constexpr int MAX_LOADS = (TILE_LOADS + NW - 1) / NW;
  static_assert(36 % CG == 0 && 16 % CG == 0 && SL % 4 == 0, "bad split");
  static_assert(!Q4 || Q8, "the q4_0 path is a variant of the quantised path");

  __shared__ __attribute__((aligned(1024))) uint8_t s_stage[kStages][STAGE_BYTES];
  // q8_0: dequantised value tile (columns 0..511, bf16, tile_unit layout)
  __shared__ __attribute__((aligned(1024))) uint8_t s_deq[Q8 ? kTile * kDL * 2 : 16];
  // q4_0: n = H (c - 8) of the tile as bf16 (576 columns, tile_unit layout)
  __shared__ __attribute__((aligned(1024))) uint8_t s_nt[Q4 ? kTile * kDK * 2 : 16];
  // partial scores per wave: bf16 path [4][64] x f32x4 in accumulator order;
  // q8_0 path as a padded 32 x 33 [head][token] matrix for the transpose
  __shared__ __attribute__((aligned(16))) float s_sx[(CG > 1 || Q8) ? NW : 1][Q8 ? 32 * 33 : 16 * 64];
  // per wave and lane: bf16 probabilities of the slice, slice max, slice sum
  __shared__ __attribute__((aligned(16))) uint32_t s_px[CG > 1 ? NW : 1][64][REC];
  __shared__ int s_pre[kMaxBatch + 1];
  __shared__ int s_misc[16];
  __shared__ int s_raise[2];

  const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
  const int hg = wave / CG, cg = wave % CG;
  const int hi = lane >> 5, l32 = lane & 31;

  // Workgroups are dispatched round-robin over the 8 XCDs; renumber them so
  // that consecutive work items (the row tiles of one part, then neighbouring
  // parts) land on the same XCD and share its L2.
  int v = blockIdx.x;
  const int G = gridDim.x;
  if ((G & 7) == 0) v = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
  const int part = v / a.m_tiles, mt = v % a.m_tiles;

  plan_prefix<NT>(a.seqlens, a.B, a.max_blocks, s_pre, s_misc);
  const int T = uniform(s_pre[a.B]);
  const int P = a.P;
  if (blockIdx.x == 0)
    for (int b = tid; b <= a.B; b += NT) a.ws_prefix[b] = s_pre[b];
  const int p_lo = part_start(part, P, T), p_hi = part_start(part + 1, P, T);

  // Sequences of this part form a contiguous range [b_first, b_last].
  if (tid == 0) s_raise[0] = s_raise[1] = 0;
  int b_first, b_last;
  part_range<NT>(s_pre, a.B, T, part == P - 1, p_lo, p_hi, s_misc, b_first, b_last);

  const int r = mt * MT + hg * 32 + l32;     // this lane's query row in its sequence
  const bool row_ok = r < a.M;
  const int q_i = row_ok ? r / a.H : 0;      // which of the s_q new tokens
  const int cbase = cg * (kDL / CG);         // first output column of this wave

  // Per-lane constant parts of the LDS operand addresses (tile_unit layout).
  // Score operand, k-step s: chunk 2s + hi of token l32 at 1024 s + kofs[s & 1].
  const int kofs0 = 16 * tile_unit(l32, hi);
  const int kofs1 = 16 * tile_unit(l32, 2 + hi) - 1024;
  const int kofsA = ((cg * KS) & 1) ? kofs1 : kofs0;   // even ks
  const int kofsB = ((cg * KS) & 1) ? kofs0 : kofs1;   // odd ks
  // Value operand, column tile ct, token half kk, read r: lane (g16, i16)
  // points at token 16 kk + 8 r + 4 h + (i16 >> 2), columns
  // cbase + 32 ct + 16 (g16 & 1) + 4 (i16 & 3) .. +3, i.e. chunk
  // cbase/8 + 4 ct + 2 (g16 & 1) + ((i16 & 3) >> 1); the chunk's (c & 3) does
  // not depend on ct, so the address is vofs[r] + 2048 ct + 256 kk.
  const int g16 = lane >> 4, i16 = lane & 15;
  const int vh = g16 >> 1, vq = i16 & 3, vs = i16 >> 2;
  const int vc = cbase / 8 + 2 * (g16 & 1) + (vq >> 1);
  const int vofs0 = 16 * tile_unit(4 * vh + vs, vc) + 8 * (vq & 1);
  const int vofs1 = 16 * tile_unit(8 + 4 * vh + vs, vc) + 8 * (vq & 1);

  // Per-lane source offsets of this wave's LDS-DMA loads within a tile.
  // bf16: load k fills units 64k .. 64k+63 = chunks 2k (lanes 0..31) and
  // 2k+1 (lanes 32..63); lane position l32 of chunk c holds token
  // l32 ^ 4(c & 3). q8_0: loads 0..17 fill the int8 rows chunk-major in
  // 16-column units (unit 32c' + t), loads 18..19 the 1152 bytes of scales.
  // q4_0: loads 0..8 fill the code rows block-major (unit 32g + t holds the
  // 32 codes of block g of token t), loads 9..10 the scales.
  uint32_t doff[MAX_LOADS];
#pragma unroll
  for (int j = 0; j < MAX_LOADS; ++j) {
    const int k = wave + NW * j;
    const int c = 2 * k + hi;
    if constexpr (!Q8) {
      doff[j] = (uint32_t)((l32 ^ (4 * (c & 3))) * kRowBytes + c * 16);
    } else {
      constexpr int RB = Q4 ? kQ4RowBytes : kQ8RowBytes;
      const int off = (k - CODE_LOADS) * 1024 + lane * 16;
      doff[j] = k < CODE_LOADS ? (uint32_t)(l32 * RB + c * 16)
                               : (uint32_t)(off < kQ8ScaleTileBytes ? off : 0);
    }
  }
  // q4_0: A operand of the Hadamard product, H[m][k] for this lane's row
  // m = l32 and columns k = 8 hi + e (first MFMA) and 16 + 8 hi + e (second)
  bf16x8 hA0, hA1;
  if constexpr (Q4) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int k0 = 8 * hi + e;
      hA0[e] = (__bf16)((__builtin_popcount(l32 & k0) & 1) ? -1.f : 1.f);
      hA1[e] = (__bf16)((__builtin_popcount(l32 & (k0 + 16)) & 1) ? -1.f : 1.f);
    }
  }

  for (int b = b_first; b <= b_last; ++b) {
    const int pre_b = uniform(s_pre[b]), pre_e = uniform(s_pre[b + 1]);
    const int L = uniform(clamp_len(((const CONST_AS int32_t*)a.seqlens)[b], a.max_blocks));
    const int seg_lo = max(p_lo, pre_b) - pre_b, seg_hi = min(p_hi, pre_e) - pre_b;
    bool split = false;
    int slot = 0;
    if (pre_e > pre_b) {
      const int fp = part_of(pre_b, P, T), lp = part_of(pre_e - 1, P, T);
      split = lp > fp;
      slot = 2 * part + ((part == fp && pre_b > p_lo) ? 1 : 0);
    }
    const int t_begin = 2 * seg_lo;
    const int t_end = min(2 * seg_hi, (L + kTile - 1) / kTile);
    const int n_tiles = max(0, t_end - t_begin);
    const CONST_AS int32_t* bt =
        (const CONST_AS int32_t*)a.block_table + (int64_t)b * a.max_blocks;

    // every block id this segment reads must be in range
    int bad_local = 0;
    for (int j = seg_lo + tid; j < seg_hi; j += NT) {
      const int id = bt[j];
      if (id < 0 || (int64_t)id >= a.num_blocks) bad_local = 1;
    }
    const bool bad = __syncthreads_or(bad_local) != 0;
    const int n_run = bad ? 0 : n_tiles;

    // absorbed query rows: operand of the score MFMA (k-steps cg*KS ..)
    bf16x8 qf[KS];
    {
      const uint16_t* qrow = a.q + ((int64_t)b * a.M + (row_ok ? r : 0)) * kDK;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int s = cg * KS + ks;
        bf16x8 z = {};
        qf[ks] = row_ok ? *reinterpret_cast<const bf16x8*>(qrow + 16 * s + 8 * hi) : z;
      }
    }
    // visible tokens of this row; padding rows see everything (never stored)
    const int n_vis = row_ok ? L - a.s_q + 1 + q_i : 0x7fffffff;

    f32x16 o[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[ct][i] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    auto issue = [&](int idx) {
      const uint32_t dst = lds_addr_of(s_stage[idx % kStages]);
      const int tt = t_begin + idx;
      const int64_t phys = bt[tt >> 1];
      if constexpr (!Q8) {
        const uint8_t* src = a.kv + (phys * kBT + (tt & 1) * kTile) * kRowBytes;
#pragma unroll
        for (int j = 0; j < MAX_LOADS; ++j) {
          const int k = wave + NW * j;
          if (k < TILE_LOADS) dma16_sbase(src, doff[j], dst + k * 1024);
        }
      } else {
        constexpr int RB = Q4 ? kQ4RowBytes : kQ8RowBytes;
        const uint8_t* src = a.kv + (phys * kBT + (tt & 1) * kTile) * RB;
        const uint8_t* ssrc =
            a.kv_scales + (phys * kBT + (tt & 1) * kTile) * kQ8ScaleRowBytes;
#pragma unroll
        for (int j = 0; j < MAX_LOADS; ++j) {
          const int k = wave + NW * j;
          if (k < CODE_LOADS)
            dma16_sbase(src, doff[j], dst + k * 1024);
          else if (k < TILE_LOADS)
            dma16_sbase(ssrc, doff[j], dst + SCALE_OFF + (k - CODE_LOADS) * 1024);
        }
      }
    };

    // wait for this wave's loads of the tile about to be consumed; at most
    // one later tile (ahead) may still be in flight
    auto wait_tile = [&](bool one_ahead) {
      if (!one_ahead) {
        wait_vmcnt<0>();
      } else if constexpr (TILE_LOADS % NW == 0) {
        wait_vmcnt<TILE_LOADS / NW>();
      } else {
        if (wave < TILE_LOADS % NW)
          wait_vmcnt<TILE_LOADS / NW + 1>();
        else
          wait_vmcnt<TILE_LOADS / NW>();
      }
    };

    // The last tile of a sequence may hold rows past its end: clear them so
    // that whatever the unused cache slots contain cannot reach the result
    // (a zero probability times a NaN would still be NaN).
    auto clear_tail = [&](LDS_AS uint8_t* st, int valid) {
      if constexpr (!Q8) {
        for (int u = tid; u < kTile * 72; u += NT) {
          const int c = u >> 5, pos = u & 31;
          if ((pos ^ (4 * (c & 3))) >= valid)
            *reinterpret_cast<LDS_AS f32x4*>(st + 16 * u) = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      } else {
        // q4_0: zero codes still mean -8; the zeroed scales make the values 0
        for (int u = tid; u < kTile * (Q4 ? 18 : 36); u += NT) {
          if ((u & 31) >= valid)
            *reinterpret_cast<LDS_AS f32x4*>(st + 16 * u) = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        for (int t = valid + tid; t < kTile; t += NT) {
          LDS_AS uint32_t* srow =
              reinterpret_cast<LDS_AS uint32_t*>(st + SCALE_OFF + t * kQ8ScaleRowBytes);
#pragma unroll
          for (int e = 0; e < kQ8ScaleRowBytes / 4; ++e) srow[e] = 0u;
        }
      }
    };

    auto compute = [&](int it, const LDS_AS uint8_t* st) {
      const int t0 = (t_begin + it) * kTile;   // first token of the tile
      // ---- (A) this wave's slice of the scores S^T (tokens x heads):
      // registers i in [SL cg, SL cg + SL), token t0 + 8(i>>2) + 4hi + (i&3)
      float tot[SL];
      if constexpr (Q8) {
      if constexpr (Q4) {
        // n = H (c - 8) for block g of all 32 tokens: two MFMAs (k = code
        // index 0..15, 16..31) of H rows against the codes as bf16(128 + c)
        // (bits 0x4300 | c), which adds 136 * sum_k H[m][k] = 4352 to row
        // m = 0 only; that is taken off. Lane (t, hi) then holds n[m][t] for
        // m = 8 q + 4 hi + (0..3), i.e. bf16 bytes 8 hi .. 8 hi + 7 of
        // chunk 4 g + q of token t in the n tile, and (g < 16) the same
        // positions of the value tile as bf16(d / sqrt(32) * n).
        auto nib8 = [](uint32_t w) {
          u32x4 r;
#pragma unroll
          for (int k = 0; k < 4; ++k)
            r[k] = ((w >> (8 * k)) & 0xFu) | (((w >> (8 * k + 4)) & 0xFu) << 16) | 0x43004300u;
          return __builtin_bit_cast(bf16x8, r);
        };
        LDS_AS uint8_t* nt = (LDS_AS uint8_t*)s_nt;
        LDS_AS uint8_t* dq = (LDS_AS uint8_t*)s_deq;
        for (int g = wave; g < 18; g += NW) {
          const LDS_AS uint8_t* cu = st + 16 * (32 * g + l32);
          const uint32_t w0 = *reinterpret_cast<const LDS_AS uint32_t*>(cu + 4 * hi);
          const uint32_t w1 = *reinterpret_cast<const LDS_AS uint32_t*>(cu + 8 + 4 * hi);
          const uint16_t sbits = *reinterpret_cast<const LDS_AS uint16_t*>(
              st + SCALE_OFF + l32 * kQ8ScaleRowBytes + 2 * g);
          const float dv = (float)__builtin_bit_cast(_Float16, sbits) * kInvSqrt32;
          const f32x16 zero = {};
          f32x16 n = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hA0, nib8(w0), zero, 0, 0, 0);
          n = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hA1, nib8(w1), n, 0, 0, 0);
          if (hi == 0) n[0] -= 4352.f;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int u = 16 * tile_unit(l32, 4 * g + q) + 8 * hi;
            *reinterpret_cast<LDS_AS uint64_t*>(nt + u) =
                (uint64_t)pack_bf16x2(n[4 * q], n[4 * q + 1]) |
                ((uint64_t)pack_bf16x2(n[4 * q + 2], n[4 * q + 3]) << 32);
            if (g < 16)
              *reinterpret_cast<LDS_AS uint64_t*>(dq + u) =
                  (uint64_t)pack_bf16x2(dv * n[4 * q], dv * n[4 * q + 1]) |
                  ((uint64_t)pack_bf16x2(dv * n[4 * q + 2], dv * n[4 * q + 3]) << 32);
          }
        }
        lds_barrier();   // every wave's blocks of the n tile are written
      } else {
        // Value tile: bf16(scale * int8) for columns 0..511.
        LDS_AS uint8_t* dq = (LDS_AS uint8_t*)s_deq;
        for (int u = tid; u < kTile * (kDL / 8); u += NT) {
          const int c = u >> 5, t = u & 31;        // 8-column chunk, token
          const uint64_t raw = *reinterpret_cast<const LDS_AS uint64_t*>(
              st + (32 * (c >> 1) + t) * 16 + 8 * (c & 1));
          const uint16_t sbits = *reinterpret_cast<const LDS_AS uint16_t*>(
              st + kQ8TileBytes + t * kQ8ScaleRowBytes + (c >> 2) * 2);
          const float sc = (float)__builtin_bit_cast(_Float16, sbits);
          bf16x8 vals;
#pragma unroll
          for (int e = 0; e < 8; ++e) vals[e] = (__bf16)(sc * (float)(int8_t)(raw >> (8 * e)));
          *reinterpret_cast<LDS_AS bf16x8*>(dq + 16 * tile_unit(t, c)) = vals;
        }
      }
        // Exact scores: S (heads x tokens, one token per lane) on the int8
        // values themselves (exact in bf16), each 32-column group's partial
        // sum times that token's fp16 scale in fp32.
        __builtin_amdgcn_sched_barrier(0);
        f32x16 snt;
#pragma unroll
        for (int i = 0; i < 16; ++i) snt[i] = 0.f;
        const LDS_AS uint8_t* srow = st + SCALE_OFF + l32 * kQ8ScaleRowBytes;
        const LDS_AS uint8_t* kraw = st + (32 * cg * KS + l32) * 16 + 8 * hi;
        // The wave's k-steps s = cg KS + ks cover columns 16s .. 16s+15; a
        // group (32 columns) is k-steps 2g, 2g+1. PAR = parity of the wave's
        // first k-step fixes, at compile time, where its groups start and end.
        // Each group accumulates from zero into one of two accumulators, and
        // is scaled into the scores one k-step after its last MFMA, so the
        // scaling never waits for the matrix core. The raw operands are read
        // two k-steps ahead.
        auto score_steps = [&](auto parc) {
          constexpr int PAR = decltype(parc)::value;
          f32x16 acc[2];
          uint64_t raw[KS];
          bf16x8 kq[KS];   // q4_0: the n-tile operands, read two k-steps ahead
          float dg[2] = {0.f, 0.f};
          auto rd4 = [&](int ks) {
            return lds_read_b128((const LDS_AS uint8_t*)s_nt + 1024 * (cg * KS + ks) +
                                 ((ks & 1) ? kofsB : kofsA));
          };
          if constexpr (Q4) {
            kq[0] = rd4(0);
            if constexpr (KS > 1) kq[1] = rd4(1);
          } else {
            raw[0] = *reinterpret_cast<const LDS_AS uint64_t*>(kraw);
            if constexpr (KS > 1) raw[1] = *reinterpret_cast<const LDS_AS uint64_t*>(kraw + 512);
          }
          auto scale_of = [&](int ks) {
            const uint16_t sbits = *reinterpret_cast<const LDS_AS uint16_t*>(
                srow + ((cg * KS + ks) >> 1) * 2);
            return (float)__builtin_bit_cast(_Float16, sbits);
          };
          auto flush = [&](int buf, float d) {
#pragma unroll
            for (int i = 0; i < 16; ++i) snt[i] += d * acc[buf][i];
          };
          // group boundaries and accumulator buffers, all known at compile time
          constexpr auto starts = [](int ks) { return ks == 0 || ((PAR + ks) & 1) == 0; };
          constexpr auto ends = [](int ks) { return ks == KS - 1 || ((PAR + ks) & 1) == 1; };
          constexpr auto buf_of = [](int ks) {
            int n = -1;
            for (int j = 0; j <= ks; ++j) n += (j == 0 || ((PAR + j) & 1) == 0) ? 1 : 0;
            return n & 1;
          };
          unroll<KS>([&](auto kc) {
            constexpr int ks = decltype(kc)::value;
            constexpr int buf = buf_of(ks);
            if constexpr (ks + 2 < KS) {
              if constexpr (Q4)
                kq[ks + 2] = rd4(ks + 2);
              else
                raw[ks + 2] = *reinterpret_cast<const LDS_AS uint64_t*>(kraw + 512 * (ks + 2));
            }
            bf16x8 kf;
            if constexpr (Q4) {
              kf = kq[ks];
            } else {
#pragma unroll
              for (int e = 0; e < 8; ++e) kf[e] = (__bf16)(float)(int8_t)(raw[ks] >> (8 * e));
            }
            if constexpr (starts(ks)) {
              const f32x16 zero = {};
              acc[buf] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[ks], kf, zero, 0, 0, 0);
              dg[buf] = scale_of(ks);
            } else {
              acc[buf] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[ks], kf, acc[buf], 0, 0, 0);
            }
            // the group that ended one k-step ago is scaled now
            if constexpr (ks > 0 && ends(ks - 1)) flush(buf_of(ks - 1), dg[buf_of(ks - 1)]);
          });
          flush(buf_of(KS - 1), dg[buf_of(KS - 1)]);
        };
        if (cg & 1)
          score_steps(std::integral_constant<int, (KS & 1)>{});
        else
          score_steps(std::integral_constant<int, 0>{});
        // transpose through LDS, summing the CG partials for this slice
        float* mine = s_sx[wave];
#pragma unroll
        for (int i = 0; i < 16; ++i) mine[(8 * (i >> 2) + 4 * hi + (i & 3)) * 33 + l32] = snt[i];
        lds_barrier();
#pragma unroll
        for (int j = 0; j < SL; ++j) {
          const int i = SL * cg + j;
          float x = 0.f;
#pragma unroll
          for (int c = 0; c < CG; ++c)
            x += s_sx[hg * CG + c][l32 * 33 + 8 * (i >> 2) + 4 * hi + (i & 3)];
          tot[j] = x;
        }
        st = (const LDS_AS uint8_t*)s_deq;
      } else {
        __builtin_amdgcn_sched_barrier(0);
        f32x16 sacc, sodd;   // two independent chains (even / odd k-steps)
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[i] = sodd[i] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int s = cg * KS + ks;
          const bf16x8 kf = lds_read_b128(st + 1024 * s + ((ks & 1) ? kofsB : kofsA));
          if (ks & 1)
            sodd = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], sodd, 0, 0, 0);
          else
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], sacc, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[i] += sodd[i];
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (CG > 1) {
          // reduce-scatter: every wave stores its partial scores, then sums
          // (in a fixed order) the partials of its own slice only
          f32x4* mine = reinterpret_cast<f32x4*>(s_sx[wave]);
#pragma unroll
          for (int q = 0; q < 4; ++q)
            mine[q * 64 + lane] = f32x4{sacc[4 * q], sacc[4 * q + 1], sacc[4 * q + 2], sacc[4 * q + 3]};
          lds_barrier();
#pragma unroll
          for (int j = 0; j < SL; ++j) tot[j] = 0.f;
#pragma unroll
          for (int c = 0; c < CG; ++c) {
            const f32x4* other = reinterpret_cast<const f32x4*>(s_sx[hg * CG + c]);
#pragma unroll
            for (int qq = 0; qq < SL / 4; ++qq) {
              const f32x4 x = other[(SL / 4 * cg + qq) * 64 + lane];
              tot[4 * qq] += x[0]; tot[4 * qq + 1] += x[1];
              tot[4 * qq + 2] += x[2]; tot[4 * qq + 3] += x[3];
            }
          }
        } else {
#pragma unroll
          for (int j = 0; j < SL; ++j) tot[j] = sacc[j];
        }
      }

      // ---- (B) softmax on the slice, against the shared reference m_run
      __builtin_amdgcn_sched_barrier(0);
      const bool interior = __all(t0 + kTile <= n_vis);
      float vv[SL];
      float smax = -INFINITY;
#pragma unroll
      for (int j = 0; j < SL; ++j) {
        const int i = SL * cg + j;
        const int tok = t0 + 8 * (i >> 2) + 4 * hi + (i & 3);
        vv[j] = (interior || tok < n_vis) ? tot[j] * a.scale_log2 : -INFINITY;
        smax = fmaxf(smax, vv[j]);
      }
      smax = fmaxf(smax, __shfl_xor(smax, 32, 64));
      float pv[SL];
      float psum = 0.f;
      auto exps = [&]() {
        psum = 0.f;
        if (m_run != -INFINITY) {
#pragma unroll
          for (int j = 0; j < SL; ++j) {
            pv[j] = __builtin_amdgcn_exp2f(vv[j] - m_run);
            psum += pv[j];
          }
        } else {
#pragma unroll
          for (int j = 0; j < SL; ++j) pv[j] = 0.f;
        }
        psum += __shfl_xor(psum, 32, 64);
      };
      exps();
      const bool raise_lane =
          smax > m_run + kRescaleThreshold || (m_run == -INFINITY && smax > -INFINITY);
      uint32_t pw[8];     // all 16 probabilities of the lane, packed bf16 pairs
      float tmax, tsum;
      if constexpr (CG > 1) {
        // all-gather the slices of the row group through LDS
        auto publish = [&]() {
          uint32_t* rec = s_px[wave][lane];
          uint32_t w[REC];
#pragma unroll
          for (int j = 0; j < SL / 2; ++j) w[j] = pack_bf16x2(pv[2 * j], pv[2 * j + 1]);
          w[SL / 2] = __builtin_bit_cast(uint32_t, smax);
          w[SL / 2 + 1] = __builtin_bit_cast(uint32_t, psum);
#pragma unroll
          for (int j = SL / 2 + 2; j < REC; ++j) w[j] = 0u;
#pragma unroll
          for (int q = 0; q < REC / 4; ++q)
            reinterpret_cast<u32x4*>(rec)[q] = u32x4{w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]};
        };
        auto gather = [&]() {
          tmax = -INFINITY;
          tsum = 0.f;
#pragma unroll
          for (int c = 0; c < CG; ++c) {
            const u32x4* rec = reinterpret_cast<const u32x4*>(s_px[hg * CG + c][lane]);
            uint32_t w[REC];
#pragma unroll
            for (int q = 0; q < REC / 4; ++q) {
              const u32x4 x = rec[q];
              w[4 * q] = x[0]; w[4 * q + 1] = x[1]; w[4 * q + 2] = x[2]; w[4 * q + 3] = x[3];
            }
#pragma unroll
            for (int j = 0; j < SL / 2; ++j) pw[(SL / 2) * c + j] = w[j];
            tmax = fmaxf(tmax, __builtin_bit_cast(float, w[SL / 2]));
            tsum += __builtin_bit_cast(float, w[SL / 2 + 1]);
          }
        };
        publish();
        if (__any(raise_lane) && lane == 0) atomicOr(&s_raise[it & 1], 1);
        lds_barrier();
        const bool rare = s_raise[it & 1] != 0;   // same value in every wave
        if (tid == 0) s_raise[(it + 1) & 1] = 0;
        gather();
        if (rare) {
          // a new reference maximum for the rows that need one; every wave
          // takes this path together (one more barrier)
          const bool raise = tmax > m_run + kRescaleThreshold ||
                             (m_run == -INFINITY && tmax > -INFINITY);
          if (__any(raise)) {
            const float m_new = tmax + kRefHeadroom;
            const float alpha = raise ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
            if (raise) m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
              for (int i = 0; i < 16; ++i) o[ct][i] *= alpha;
          }
          exps();
          lds_barrier();       // everyone has read the old records
          publish();
          lds_barrier();
          gather();
        }
      } else {
        tmax = smax;
        if (__builtin_expect(__any(raise_lane), 0)) {
          const bool raise = raise_lane;
          const float m_new = tmax + kRefHeadroom;
          const float alpha = raise ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
          if (raise) m_run = m_new;
          l_run *= alpha;
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[ct][i] *= alpha;
          exps();
        }
        tsum = psum;
#pragma unroll
        for (int j = 0; j < 8; ++j) pw[j] = pack_bf16x2(pv[2 * j], pv[2 * j + 1]);
      }
      l_run += tsum;
      const bf16x8 pb0 = __builtin_bit_cast(bf16x8, u32x4{pw[0], pw[1], pw[2], pw[3]});
      const bf16x8 pb1 = __builtin_bit_cast(bf16x8, u32x4{pw[4], pw[5], pw[6], pw[7]});

      // ---- (C) value product O^T (columns x heads) += V^T P^T
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const bf16x8 v0 = vt_fragment(st + vofs0 + 2048 * ct, st + vofs1 + 2048 * ct);
        o[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v0, pb0, o[ct], 0, 0, 0);
        const bf16x8 v1 =
            vt_fragment(st + vofs0 + 2048 * ct + 256, st + vofs1 + 2048 * ct + 256);
        o[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v1, pb1, o[ct], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    };

    // 3-stage ring: tiles it+1 and it+2 load while tile it is consumed.
    // Everything the compiler itself loaded (the query rows) is drained first,
    // so its own wait counts stay exact while DMAs are in flight.
    wait_vmcnt<0>();
    if (n_run > 0) issue(0);
    if (n_run > 1) issue(1);
    for (int it = 0; it < n_run; ++it) {
      wait_tile(it + 1 < n_run);
      lds_barrier();
      if (it + 2 < n_run) issue(it + 2);
      LDS_AS uint8_t* st = (LDS_AS uint8_t*)s_stage[it % kStages];
      const int valid = L - (t_begin + it) * kTile;
      if (valid < kTile) {           // last tile of the sequence
        clear_tail(st, valid);
        lds_barrier();
      }
      compute(it, st);
    }

    // ---- epilogue: final rows, or bf16 partials of a split sequence
    const float inv_l = l_run > 0.f ? 1.f / l_run : 0.f;
    float lse_v = l_run > 0.f ? (m_run + __log2f(l_run)) * 0.69314718055994531f : -INFINITY;
    if (bad) lse_v = __builtin_nanf("");
    if (row_ok) {
      const int64_t row = (int64_t)b * a.M + r;
      if (!split) {
        uint16_t* orow = a.out + row * kDL;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int col = cbase + 32 * ct + 8 * g + 4 * hi;
            uint16_t hbits[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
              hbits[e] = bad ? (uint16_t)0x7FC0 : f32_to_bf16_bits(o[ct][4 * g + e] * inv_l);
            const uint64_t packed = (uint64_t)hbits[0] | ((uint64_t)hbits[1] << 16) |
                                    ((uint64_t)hbits[2] << 32) | ((uint64_t)hbits[3] << 48);
            *reinterpret_cast<uint64_t*>(orow + col) = packed;
          }
        if (hi == 0 && cg == 0) a.lse[row] = lse_v;
      } else {
        uint16_t* prow = a.part_o + ((int64_t)slot * a.M + r) * kDL;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int col = cbase + 32 * ct + 8 * g + 4 * hi;
            uint32_t w0, w1;
            if (bad) {
              w0 = w1 = 0x7FC07FC0u;
            } else {
              w0 = pack_bf16x2(o[ct][4 * g + 0] * inv_l, o[ct][4 * g + 1] * inv_l);
              w1 = pack_bf16x2(o[ct][4 * g + 2] * inv_l, o[ct][4 * g + 3] * inv_l);
            }
            *reinterpret_cast<uint64_t*>(prow + col) = (uint64_t)w0 | ((uint64_t)w1 << 32);
          }
        if (hi == 0 && cg == 0) a.part_lse[(int64_t)slot * a.M + r] = lse_v;
      }
    }
    wait_vmcnt<0>();
    __syncthreads();   // the ring is reused by the next sequence
  }
}


// acc *= alpha in place on the accumulation registers (rare path of the
// online softmax). Done in asm so that the accumulators of the value product
// keep a single home in AGPRs; compiler-generated VALU scaling would make the
// allocator stage every accumulator through VGPRs on each loop iteration.
// The leading nops cover the MFMA-write -> accvgpr-read latency.
__device__ __forceinline__ void acc_scale(f32x16& acc, float alpha) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" ::: "memory");
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float x = acc[i];
    float t;
    asm volatile(
        "v_accvgpr_read_b32 %1, %0\n\t"
        "v_mul_f32 %1, %1, %2\n\t"
        "v_accvgpr_write_b32 %0, %1"
        : "+a"(x), "=&v"(t)
        : "v"(alpha));
    acc[i] = x;
  }
}

// The same for a 4-register accumulator (16x16 MFMA).
__device__ __forceinline__ void acc_scale4(f32x4& acc, float alpha) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" ::: "memory");
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float x = acc[i];
    float t;
    asm volatile(
        "v_accvgpr_read_b32 %1, %0\n\t"
        "v_mul_f32 %1, %1, %2\n\t"
        "v_accvgpr_write_b32 %0, %1"
        : "+a"(x), "=&v"(t)
        : "v"(alpha));
    acc[i] = x;
  }
}

// Row-group tile layout of the 128-row kernel: block 4 C + R (1 KiB) holds
// tokens 8R..8R+7 and chunks 8C..8C+7 (16-byte units); token 8R + r, chunk
// 8C + c sits in its block at unit (r & 3) | ((r >> 2) ^ c) & 1) << 2 |
// ((R ^ (c >> 1)) & 1) << 3 | (c & 1) << 4 | (c >> 2 & 1) << 5. Every LDS-DMA
// copy fills one block from eight whole 128-byte lines, and the score reads
// (32 tokens x two chunks) and the transposing value reads (4 tokens x 4
// chunks per 32 lanes) each hit distinct 16-byte bank groups.
__device__ __forceinline__ int rg_unit(int t, int c) {
  const int R = t >> 3, r = t & 7, C = c >> 3, cc = c & 7;
  return 64 * (4 * C + R) + ((r & 3) | ((((r >> 2) ^ cc) & 1) << 2) |
                             (((R ^ (cc >> 1)) & 1) << 3) | ((cc & 1) << 4) |
                             (((cc >> 2) & 1) << 5));
}
// Byte offset of score k-step k (chunks 2k, 2k+1) that does not depend on
// the lane.
__device__ __forceinline__ constexpr int kstep_ofs(int k) { return 4096 * (k >> 2) + 512 * ((k >> 1) & 1); }

// ------------------------------------------------- bf16 decode kernel (rows)

// One workgroup = 4 waves (one per SIMD) on one KV partition for a tile of
// 32*HG query rows. Every wave owns whole query rows: wave (hg, cg) computes
// the complete 576-column scores of its 32-row group hg, so no partial score
// ever crosses waves, and the value product of those rows for output columns
// [cg*512/CG, (cg+1)*512/CG), CG = 4/HG. With HG = 4 nothing is computed
// twice; with fewer row groups (short rows per sequence) the CG waves of a
// group repeat the same score product, which costs MFMA time these
// bandwidth-bound shapes have to spare.
//
// Per 32-token tile the only workgroup synchronisation is one barrier: a
// 4-stage LDS ring holds the tile whose value product runs, the tile whose
// scores run, and two tiles in flight. The score product of tile i+1 is
// issued before the softmax of tile i, so the exponentials overlap MFMA work
// of the same wave.
template <int HG, bool NTC>
__global__ __launch_bounds__(256, 1) void mla_decode_rows_kernel(DecodeParams a) {
  constexpr int NW = 4;
  constexpr int NT = 64 * NW;
  constexpr int CG = NW / HG;             // waves per row group
  constexpr int MT = 32 * HG;             // query rows per workgroup
  constexpr int NCT = 16 / CG;            // 32-column output blocks per wave
  constexpr int NST = 4;                  // ring stages
  constexpr int LPW = 36 / NW;            // 1 KiB LDS-DMA loads per wave per tile
  // HG = 4: 128 rows per CU leave no registers for a second score tile, so
  // the score product of a tile is not overlapped with the previous softmax
  constexpr bool PIPE = HG != 4;
  constexpr int KPF = HG == 4 ? 2 : 3;    // score operands in flight
  constexpr int VPF = HG == 4 ? 2 : 3;    // value operands in flight
  static_assert(HG == 1 || HG == 2 || HG == 4, "row groups");

  __shared__ __attribute__((aligned(1024))) uint8_t s_stage[NST][kTileBytes];
  __shared__ int s_pre[kMaxBatch + 1];
  __shared__ int s_misc[16];

  const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
  const int hg = wave / CG, cg = wave % CG;
  const int hi = lane >> 5, l32 = lane & 31;

  int v = blockIdx.x;
  const int G = gridDim.x;
  if ((G & 7) == 0) v = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
  const int part = v / a.m_tiles, mt = v % a.m_tiles;

  plan_prefix<NT>(a.seqlens, a.B, a.max_blocks, s_pre, s_misc);
  const int T = uniform(s_pre[a.B]);
  const int P = a.P;
  if (blockIdx.x == 0)
    for (int b = tid; b <= a.B; b += NT) a.ws_prefix[b] = s_pre[b];
  const int p_lo = part_start(part, P, T), p_hi = part_start(part + 1, P, T);
  int b_first, b_last;
  part_range<NT>(s_pre, a.B, T, part == P - 1, p_lo, p_hi, s_misc, b_first, b_last);

  const int r = mt * MT + hg * 32 + l32;     // this lane's query row in its sequence
  const bool row_ok = r < a.M;
  const int q_i = row_ok ? r / a.H : 0;
  const int cbase = cg * (kDL / CG);         // first output column of this wave

  // Tiles use the row-group layout of the 128-row kernel (rg_unit): score
  // operand of k-step s (chunk 2s + hi of token l32) at byte
  // kstep_ofs(s) + (s odd ? kofs1 : kofs0).
  const int kR = l32 >> 3, kr = l32 & 7;
  const int kpart = 1024 * kR + 16 * ((kr & 3) | ((((kr >> 2) ^ hi) & 1) << 2) | (hi << 4));
  const int kofs0 = kpart + 128 * (kR & 1);
  const int kofs1 = kpart + 128 * ((kR & 1) ^ 1);
  // Value operand: lane (g16, i16) of column block ct, token half kk points
  // at token 16 kk + 4 (g16 >> 1) + (i16 >> 2) (+8 for the second read),
  // columns cbase + 32 ct + 16 (g16 & 1) + 4 (i16 & 3) .. +3: byte
  // vofs{0,1} + vct_ofs(ct) + 2048 kk.
  const int g16 = lane >> 4, i16 = lane & 15;
  const int vh = g16 >> 1, vq = i16 & 3, vs = i16 >> 2;
  const int vlane = 64 * cbase + 16 * vs + 64 * (vh ^ (vq >> 1)) + 256 * (vq >> 1) + 8 * (vq & 1);
  const int vofs0 = vlane + 128 * (g16 & 1);
  const int vofs1 = vlane + 1024 + 128 * ((g16 & 1) ^ 1);
  // LDS-DMA: copy j of wave w fills block 4 j + w from eight whole 128-byte
  // lines (as in the 128-row kernel).
  const int dc0 = (lane >> 4) & 1;
  const int dr = (lane & 3) | ((((lane >> 2) & 1) ^ dc0) << 2);
  const int dcc = dc0 | ((((lane >> 3) ^ wave) & 1) << 1) | (((lane >> 5) & 1) << 2);
  const uint32_t doff = (uint32_t)((8 * wave + dr) * kRowBytes + 16 * dcc);
  auto copy = [](const void* src, uint32_t off, uint32_t dst) {
    if constexpr (NTC)
      dma16_sbase_nt(src, off, dst);
    else
      dma16_sbase(src, off, dst);
  };
  auto vct_ofs = [](int ct) { return 4096 * (ct >> 1) + 512 * (ct & 1); };

  for (int b = b_first; b <= b_last; ++b) {
    const int pre_b = uniform(s_pre[b]), pre_e = uniform(s_pre[b + 1]);
    const int L = uniform(clamp_len(((const CONST_AS int32_t*)a.seqlens)[b], a.max_blocks));
    const int seg_lo = max(p_lo, pre_b) - pre_b, seg_hi = min(p_hi, pre_e) - pre_b;
    bool split = false;
    int slot = 0;
    if (pre_e > pre_b) {
      const int fp = part_of(pre_b, P, T), lp = part_of(pre_e - 1, P, T);
      split = lp > fp;
      slot = 2 * part + ((part == fp && pre_b > p_lo) ? 1 : 0);
    }
    const int t_begin = 2 * seg_lo;
    const int t_end = min(2 * seg_hi, (L + kTile - 1) / kTile);
    const int n_tiles = max(0, t_end - t_begin);
    const CONST_AS int32_t* bt =
        (const CONST_AS int32_t*)a.block_table + (int64_t)b * a.max_blocks;

    int bad_local = 0;
    for (int j = seg_lo + tid; j < seg_hi; j += NT) {
      const int id = bt[j];
      if (id < 0 || (int64_t)id >= a.num_blocks) bad_local = 1;
    }
    const bool bad = __syncthreads_or(bad_local) != 0;
    const int n_run = bad ? 0 : n_tiles;

    bf16x8 qf[36];
    {
      const uint16_t* qrow = a.q + ((int64_t)b * a.M + (row_ok ? r : 0)) * kDK;
      const uint32_t sg = a.q_sign2;
#pragma unroll
      for (int s = 0; s < 36; ++s) {
        u32x4 z = {0u, 0u, 0u, 0u};
        if (row_ok) z = *reinterpret_cast<const u32x4*>(qrow + 16 * s + 8 * hi) ^ sg;
        qf[s] = __builtin_bit_cast(bf16x8, z);
      }
    }
    const int n_vis = row_ok ? L - a.s_q + 1 + q_i : 0x7fffffff;

    f32x16 o[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[ct][i] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    // Block id of a tile, read one issue ahead (a scalar load whose latency
    // then hides behind a whole iteration); indices past the segment reuse
    // its last tile.
    auto block_of = [&](int idx) {
      return bt[(t_begin + min(idx, n_run - 1)) >> 1];
    };
    int next_phys = 0;
    auto issue = [&](int idx) {
      const uint32_t dst = lds_addr_of(s_stage[idx % NST]) + 1024 * wave;
      const int tt = t_begin + idx;
      const int64_t phys = next_phys;
      next_phys = block_of(idx + 1);
      const uint8_t* src = a.kv + (phys * kBT + (tt & 1) * kTile) * kRowBytes;
#pragma unroll
      for (int j = 0; j < LPW; ++j) copy(src + 128 * j, doff, dst + 4096 * j);
    };

    // Rows past the end of the sequence in its last tile are cleared, so that
    // whatever unused cache slots hold cannot reach the result.
    auto clear_tail = [&](LDS_AS uint8_t* st, int valid) {
      for (int u = tid; u < kTile * 72; u += NT) {
        const int c0 = (u >> 4) & 1;
        const int token = 8 * ((u >> 6) & 3) + ((u & 3) | ((((u >> 2) & 1) ^ c0) << 2));
        if (token >= valid)
          *reinterpret_cast<LDS_AS f32x4*>(st + 16 * u) = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    };

    // S^T (tokens x rows) of one tile: register i is token 8(i>>2) + 4hi + (i&3)
    auto scores = [&](const LDS_AS uint8_t* st) {
      f32x16 acc;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = 0.f;
      auto rd = [&](int s) { return lds_read_b128(st + kstep_ofs(s) + ((s & 1) ? kofs1 : kofs0)); };
      constexpr int D = 4;
      bf16x8 kf[D];
#pragma unroll
      for (int j = 0; j < D; ++j) kf[j] = rd(j);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int s = 0; s < 36; ++s) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s % D], qf[s], acc, 0, 0, 0);
        if (s + D < 36) kf[s % D] = rd(s + D);
        __builtin_amdgcn_sched_barrier(0);
      }
      return acc;
    };

    auto prepare = [&](int idx) {   // tile idx has landed in every wave's share
      const int valid = L - (t_begin + idx) * kTile;
      if (valid < kTile) {
        clear_tail((LDS_AS uint8_t*)s_stage[idx % NST], valid);
        lds_barrier();
      }
    };

    f32x16 s_cur;
    wait_vmcnt<0>();
    if (n_run > 0) next_phys = block_of(0);
    if (n_run > 0) issue(0);
    if (n_run > 1) issue(1);
    if (n_run > 2) issue(2);
    if (PIPE && n_run > 0) {
      if (n_run > 2) wait_vmcnt<2 * LPW>();
      else if (n_run > 1) wait_vmcnt<LPW>();
      else wait_vmcnt<0>();
      lds_barrier();
      prepare(0);
      s_cur = scores((const LDS_AS uint8_t*)s_stage[0]);
    }
    for (int it = 0; it < n_run; ++it) {
      if (PIPE) {
        if (it + 1 < n_run) {
          if (it + 2 < n_run) wait_vmcnt<LPW>();
          else wait_vmcnt<0>();
          lds_barrier();
          if (it + 3 < n_run) issue(it + 3);
          prepare(it + 1);
        }
      } else {
        // tile it landed; tiles it+1, it+2 may still be in flight
        if (it + 2 < n_run) wait_vmcnt<2 * LPW>();
        else if (it + 1 < n_run) wait_vmcnt<LPW>();
        else wait_vmcnt<0>();
        lds_barrier();
        if (it + 3 < n_run) issue(it + 3);
        prepare(it);
        s_cur = scores((const LDS_AS uint8_t*)s_stage[it % NST]);
      }
      // One straight-line block, software-pipelined by hand: the score product
      // of tile it+1 (on the last tile a dummy pass over a resident stage,
      // result unused), with three LDS operand reads in flight, and between
      // its MFMAs the softmax of tile it, assuming its reference maximum holds.
      // Interior tiles (every token visible to every row) skip the mask.
      const LDS_AS uint8_t* sn = (const LDS_AS uint8_t*)s_stage[(it + 1) % NST];
      const int t0 = (t_begin + it) * kTile;
      const float c = a.scale_mag_log2;
      const float neg_m = m_run == -INFINITY ? 0.f : -m_run;
      float x[16];
      float lmax, psum;
      uint32_t pw[8];
      f32x16 s_next;
      auto kread = [&](int s) {
        return lds_read_b128(sn + kstep_ofs(s) + ((s & 1) ? kofs1 : kofs0));
      };
      // x[i]: the raw score (interior tiles) or the scaled, masked score;
      // kept so that the rare path can redo the probabilities
      auto fused = [&](auto masked_tag) {
        constexpr bool MASKED = decltype(masked_tag)::value;
        // visible tokens of this lane's row within the tile, minus the lane's
        // token offset 4 hi (masked tiles only)
        const int lim = n_vis - t0 - 4 * hi;
#pragma unroll
        for (int i = 0; i < 16; ++i) s_next[i] = 0.f;
        float mx[4];
        float p_prev = 0.f;
        psum = 0.f;
        bf16x8 kb[KPF];
        if (PIPE) {
#pragma unroll
          for (int j = 0; j < KPF; ++j) kb[j] = kread(j);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < 36; ++s) {
          if (PIPE) {
            s_next = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb[s % KPF], qf[s], s_next, 0, 0, 0);
            if (s + KPF < 36) kb[s % KPF] = kread(s + KPF);
          }
          if (s < 16) {
            // masked tiles scale first and then select, so that a masked
            // token is -inf whatever the scale (even 0)
            const int i = s;
            x[i] = MASKED ? ((8 * (i >> 2) + (i & 3) < lim) ? s_cur[i] * c : -INFINITY) : s_cur[i];
            if ((i & 3) == 3)
              mx[i >> 2] = fmaxf(fmaxf(x[i - 3], x[i - 2]), fmaxf(x[i - 1], x[i]));
          } else if (s < 32) {
            const int i = s - 16;
            const float pi = __builtin_amdgcn_exp2f(MASKED ? x[i] + neg_m : __builtin_fmaf(x[i], c, neg_m));
            psum += pi;
            if (i & 1) pw[i >> 1] = pack_bf16x2(p_prev, pi);
            p_prev = pi;
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        lmax = fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3]));
        if (!MASKED) lmax *= c;
      };
      const bool masked = !__all(t0 + kTile <= n_vis);
      if (!masked)
        fused(std::integral_constant<bool, false>{});
      else
        fused(std::integral_constant<bool, true>{});

      if (__builtin_expect(__any(lmax > m_run + kRescaleThreshold), 0)) {
        // a new reference maximum: the two lanes holding a row's tokens agree
        // on it, the accumulators are rescaled, the probabilities redone
        const float rmax = fmaxf(lmax, __shfl_xor(lmax, 32, 64));
        const bool raise = rmax > m_run + kRescaleThreshold;
        const float m_new = rmax + kRefHeadroom;
        const float alpha = raise ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
        if (__any(raise && m_run != -INFINITY)) {
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) acc_scale(o[ct], alpha);
        }
        l_run *= alpha;
        if (raise) m_run = m_new;
        const float neg_m2 = m_run == -INFINITY ? 0.f : -m_run;
        psum = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float p0 = __builtin_amdgcn_exp2f(masked ? x[2 * j] + neg_m2
                                                         : __builtin_fmaf(x[2 * j], c, neg_m2));
          const float p1 = __builtin_amdgcn_exp2f(masked ? x[2 * j + 1] + neg_m2
                                                         : __builtin_fmaf(x[2 * j + 1], c, neg_m2));
          psum += p0 + p1;
          pw[j] = pack_bf16x2(p0, p1);
        }
      }
      l_run += psum;
      const bf16x8 pb[2] = {__builtin_bit_cast(bf16x8, u32x4{pw[0], pw[1], pw[2], pw[3]}),
                            __builtin_bit_cast(bf16x8, u32x4{pw[4], pw[5], pw[6], pw[7]})};

      // ---- value product O^T (columns x rows) += V^T P^T of tile it, token
      // half major so consecutive MFMAs are independent; operands of two
      // steps ahead in flight
      const LDS_AS uint8_t* st = (const LDS_AS uint8_t*)s_stage[it % NST];
      auto vread = [&](int q) {
        const int ct = q % NCT, kk = q / NCT;
        const int o = vct_ofs(ct) + 2048 * kk;
        return vt_fragment(st + vofs0 + o, st + vofs1 + o);
      };
      constexpr int NQ = 2 * NCT;
      bf16x8 va[VPF];
#pragma unroll
      for (int j = 0; j < VPF; ++j) va[j] = vread(j);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        o[q % NCT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[q % VPF], pb[q / NCT], o[q % NCT], 0, 0, 0);
        if (q + VPF < NQ) va[q % VPF] = vread(q + VPF);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (PIPE) s_cur = s_next;
    }

    // ---- epilogue: final rows, or bf16 partials of a split sequence
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    const float inv_l = l_tot > 0.f ? 1.f / l_tot : 0.f;
    float lse_v = l_tot > 0.f ? (m_run + __log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
    if (bad) lse_v = __builtin_nanf("");
    if (row_ok) {
      const int64_t row = (int64_t)b * a.M + r;
      if (!split) {
        uint16_t* orow = a.out + row * kDL;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int col = cbase + 32 * ct + 8 * g + 4 * hi;
            uint16_t hbits[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
              hbits[e] = bad ? (uint16_t)0x7FC0 : f32_to_bf16_bits(o[ct][4 * g + e] * inv_l);
            const uint64_t packed = (uint64_t)hbits[0] | ((uint64_t)hbits[1] << 16) |
                                    ((uint64_t)hbits[2] << 32) | ((uint64_t)hbits[3] << 48);
            *reinterpret_cast<uint64_t*>(orow + col) = packed;
          }
        if (hi == 0 && cg == 0) a.lse[row] = lse_v;
      } else {
        uint16_t* prow = a.part_o + ((int64_t)slot * a.M + r) * kDL;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int col = cbase + 32 * ct + 8 * g + 4 * hi;
            uint32_t w0, w1;
            if (bad) {
              w0 = w1 = 0x7FC07FC0u;
            } else {
              w0 = pack_bf16x2(o[ct][4 * g + 0] * inv_l, o[ct][4 * g + 1] * inv_l);
              w1 = pack_bf16x2(o[ct][4 * g + 2] * inv_l, o[ct][4 * g + 3] * inv_l);
            }
            *reinterpret_cast<uint64_t*>(prow + col) = (uint64_t)w0 | ((uint64_t)w1 << 32);
          }
        if (hi == 0 && cg == 0) a.part_lse[(int64_t)slot * a.M + r] = lse_v;
      }
    }
    wait_vmcnt<0>();
    __syncthreads();   // the ring is reused by the next sequence
  }
}

// ------------------------------------------- bf16 decode kernel (16-row tile)

// For at most 16 query rows per sequence (16 heads and one query token, or 8
// heads and two): the rows fit the N side of v_mfma_f32_16x16x32_bf16, so no
// padded rows reach the matrix cores, and the query fragments of a wave take
// 20 VGPRs. Wave w:
//  * computes partial scores S^T (32 tokens x 16 rows) of a tile over its
//    share of the 576-column contraction: k-steps of 32 columns 0-4, 5-9,
//    10-13, 14-17;
//  * after one barrier, sums the four partials from LDS (in the same order in
//    every wave, so all waves hold the same scores) and runs the online
//    softmax on them: per lane, 8 tokens of one row;
//  * accumulates the value product O^T += V^T P^T for output columns
//    128w..128w+127; the probabilities are already its B operand (token
//    order permuted, with the V^T operand read in the same order).
// The tile stream does not stop at a sequence boundary: the first three tiles
// of the next segment are issued while the current one finishes, block ids
// are loaded two segments ahead and query fragments one segment ahead, so a
// boundary costs one drain of the memory counter (after the output stores)
// instead of a chain of dependent loads.
struct NarrowSeg {
  int b, L, pre_e, seg_lo, seg_len, t_begin, n, slot;
  bool split;
};

__global__ __launch_bounds__(256, 1) void mla_decode_narrow_kernel(DecodeParams a) {
  constexpr int NW = 4;
  constexpr int NT = 64 * NW;
  constexpr int MT = 16;                  // query rows per workgroup
  constexpr int NST = 4;                  // ring stages
  constexpr int LPW = 36 / NW;            // 1 KiB LDS-DMA loads per wave per tile
  constexpr int KQ = 5;                   // k-steps of a wave (at most)

  __shared__ __attribute__((aligned(1024))) uint8_t s_stage[NST][kTileBytes];
  __shared__ __attribute__((aligned(16))) f32x4 s_x[NW][2][64];   // partial scores
  // plan scratch, inside ring stage 3 until the first tile is issued
  int* s_pre = reinterpret_cast<int*>(s_stage[3]);
  int* s_misc = reinterpret_cast<int*>(s_stage[3] + 4 * (kMaxBatch + 8));

  const int tid = threadIdx.x, wave = uniform(tid >> 6);
  const int lane = tid & 63, i16 = lane & 15, g = lane >> 4;

  int v = blockIdx.x;
  const int G = gridDim.x;
  if ((G & 7) == 0) v = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
  const int part = v / a.m_tiles, mt = v % a.m_tiles;

  plan_prefix<NT>(a.seqlens, a.B, a.max_blocks, s_pre, s_misc);
  const int T = uniform(s_pre[a.B]);
  const int P = a.P;
  if (blockIdx.x == 0)
    for (int b = tid; b <= a.B; b += NT) a.ws_prefix[b] = s_pre[b];
  const int p_lo = part_start(part, P, T), p_hi = part_start(part + 1, P, T);
  int b_first, b_last;
  part_range<NT>(s_pre, a.B, T, part == P - 1, p_lo, p_hi, s_misc, b_first, b_last);
  const int pre_first = b_first <= b_last ? uniform(s_pre[b_first]) : 0;
  __syncthreads();   // ring stage 3 is free from here on
  if (b_first > b_last) return;

  // ---- per-lane constants
  const int r = mt * MT + i16;               // query row of this lane
  const bool row_ok = r < a.M;
  const int q_i = row_ok ? r / a.H : 0;
  const int ks0 = 4 * wave + min(wave, 2);   // first k-step of this wave
  const bool five = wave < 2;                // waves 0, 1 take five k-steps
  // Tile layout of this kernel (row groups): the tile is cut into 36 blocks
  // of 8 tokens x 8 chunks (16-byte units, 8 columns each), block
  // 4 C + R holding tokens 8R..8R+7 and chunks 8C..8C+7 at 1 KiB per block.
  // Inside a block, token 8R + r and chunk 8C + c sit at unit
  // r | ((R ^ c) & 1) << 3 | (c >> 1) << 4 (c taken mod 8). One LDS-DMA copy
  // fills one block from eight whole 128-byte lines, so the copies can use the
  // non-temporal policy; the reads below touch 16 (score) or 32 (value)
  // different 16-byte bank groups per access, i.e. no bank conflicts.
  //
  // Score operand (A, tokens x columns): token 16 tb + i16, columns
  // 32 ks + 8 g .. +7 (chunk 4 ks + g): byte 4096 (ks >> 1) + 512 (ks & 1)
  // + kofs; tb = 1 adds 2048.
  const int kofs = 1024 * (i16 >> 3) + 16 * (i16 & 7) + 128 * ((i16 >> 3) ^ (g & 1)) +
                   256 * (g >> 1);
  // Value operand (A, columns x tokens), transposing reads: lane 4 s + q of
  // group g points at token 4 g + s (+16 for the second read), columns
  // 128 w + 16 ct + 4 q .. +3, i.e. chunk 16 w + 2 ct + (q >> 1): byte
  // vb[h] + 4096 (ct >> 2) + 256 (ct & 3).
  const int vs = i16 >> 2, vq = i16 & 3;
  int vb[2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
    vb[h] = 8192 * wave + 2048 * h + 1024 * (g >> 1) + 16 * (4 * (g & 1) + vs) +
            128 * ((g >> 1) ^ (vq >> 1)) + 8 * (vq & 1);
  // LDS-DMA: copy j of wave w fills block 4 j + w (tokens 8w..8w+7, chunks
  // 8j..8j+7); lane l takes token 8w + (l & 7), chunk 8j + c with
  // c = 2 (l >> 4) + (((l >> 3) ^ w) & 1), which lands at unit l of the block.
  const uint32_t doff = (uint32_t)((8 * wave + (lane & 7)) * kRowBytes +
                                   16 * (2 * (lane >> 4) + (((lane >> 3) ^ wave) & 1)));

  // ---- segments: the part's share of sequences b_first .. b_last
  auto make_seg = [&](int b, int pre_b) {
    NarrowSeg s;
    s.b = b;
    if (b > b_last) {
      s.L = 0; s.pre_e = pre_b; s.seg_lo = 0; s.seg_len = 0; s.t_begin = 0; s.n = 0;
      s.slot = 0; s.split = false;
      return s;
    }
    s.L = uniform(clamp_len(((const CONST_AS int32_t*)a.seqlens)[b], a.max_blocks));
    s.pre_e = pre_b + (s.L + kBT - 1) / kBT;
    s.seg_lo = max(p_lo, pre_b) - pre_b;
    const int seg_hi = min(p_hi, s.pre_e) - pre_b;
    s.seg_len = max(0, seg_hi - s.seg_lo);
    s.split = false;
    s.slot = 0;
    if (s.pre_e > pre_b) {
      const int fp = part_of(pre_b, P, T), lp = part_of(s.pre_e - 1, P, T);
      s.split = lp > fp;
      s.slot = 2 * part + ((part == fp && pre_b > p_lo) ? 1 : 0);
    }
    s.t_begin = 2 * s.seg_lo;
    const int t_end = min(2 * seg_hi, (s.L + kTile - 1) / kTile);
    // an empty pool has no block to stand in for invalid ids: nothing is
    // streamed and the id check poisons the segment
    s.n = a.num_blocks > 0 ? max(0, t_end - s.t_begin) : 0;
    return s;
  };
  // Block ids base .. base+63 of a segment, one per lane (the last one
  // repeated past the end). Checked once landed: an id outside
  // [0, num_blocks) poisons the segment (NaN output and lse) and is replaced
  // by block 0, so that no copy ever leaves the cache.
  auto load_ids = [&](const NarrowSeg& s, int base) {
    if (s.seg_len == 0) return 0;
    const int j = base + min(lane, max(0, s.seg_len - base - 1));
    return ((const int32_t*)a.block_table)[(int64_t)s.b * a.max_blocks + s.seg_lo + j];
  };
  auto check_ids = [&](const NarrowSeg& s, int base, int& ids, bool& bad) {
    const bool inval = ids < 0 || (int64_t)ids >= a.num_blocks;
    bad = bad || __any(inval && base + lane < s.seg_len);
    ids = inval ? 0 : ids;
  };
  auto load_q = [&](const NarrowSeg& s, u32x4* dst) {
    if (s.b > b_last) return;
    const uint16_t* qrow = a.q + ((int64_t)s.b * a.M + (row_ok ? r : 0)) * kDK + 8 * g;
#pragma unroll
    for (int j = 0; j < KQ; ++j)
      dst[j] = *reinterpret_cast<const u32x4*>(qrow + 32 * min(ks0 + j, 17));
  };

  NarrowSeg sc = make_seg(b_first, pre_first);
  NarrowSeg sn = make_seg(b_first + 1, sc.pre_e);
  int ids_c = load_ids(sc, 0), ids_n = load_ids(sn, 0), ids_nn = 0;
  bool bad_c = false, bad_n = false, bad_nn = false;
  u32x4 qn[KQ];
  load_q(sc, qn);
  wait_vmcnt<0>();
  check_ids(sc, 0, ids_c, bad_c);
  check_ids(sn, 0, ids_n, bad_n);

  int g_base = 0;   // stream index of the current segment's first tile
  int iss = 0;      // tiles issued so far (stream order)
  int bt_base = 0;  // first block of the current segment's id window
  // Next tile of the stream: the current segment's, then at most three of the
  // next segment's.
  auto issuable = [&]() { return iss < g_base + sc.n + min(sn.n, 3); };
  // Source and ring slot of the next tile of the stream; advances the stream.
  auto next_tile = [&](const uint8_t*& src, uint32_t& dst) {
    const int rel = iss - g_base;
    int64_t phys;
    int half;
    if (rel < sc.n) {
      int rb = (rel >> 1) - bt_base;
      if (rb >= 64) {
        bt_base += 64;
        rb -= 64;
        ids_c = load_ids(sc, bt_base);
        wait_vmcnt<0>();
        check_ids(sc, bt_base, ids_c, bad_c);
      }
      phys = uniform(__builtin_amdgcn_readlane(ids_c, rb));
      half = rel & 1;
    } else {
      const int idx = rel - sc.n;
      phys = uniform(__builtin_amdgcn_readlane(ids_n, idx >> 1));
      half = idx & 1;
    }
    src = a.kv + (phys * kBT + half * kTile) * kRowBytes;
    dst = lds_addr_of(s_stage[iss % NST]) + 1024 * wave;
    ++iss;
  };
  auto issue_one = [&]() {
    const uint8_t* src;
    uint32_t dst;
    next_tile(src, dst);
#pragma unroll
    for (int j = 0; j < LPW; ++j) dma16_sbase_nt(src + 128 * j, doff, dst + 4096 * j);
  };
  // Tokens past the end of the sequence in its last tile are cleared, so that
  // whatever unused cache slots hold cannot reach the value product.
  auto clear_tail = [&](LDS_AS uint8_t* st, int valid) {
    for (int u = tid; u < kTile * 72; u += NT) {
      const int token = 8 * ((u >> 6) & 3) + (u & 7);
      if (token >= valid)
        *reinterpret_cast<LDS_AS f32x4*>(st + 16 * u) = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };

  for (int b = b_first; b <= b_last; ++b) {
    // Here every earlier memory operation has completed: the query rows of
    // this segment are in qn, its first id window in ids_c (checked), and
    // the next segment's in ids_n (checked).
    bf16x8 qf[KQ];
    {
      const uint32_t sg = row_ok ? a.q_sign2 : 0u;
      const uint32_t keep = row_ok ? 0xffffffffu : 0u;
#pragma unroll
      for (int j = 0; j < KQ; ++j) qf[j] = __builtin_bit_cast(bf16x8, (qn[j] ^ sg) & keep);
    }
    const NarrowSeg snn = make_seg(b + 2, sn.pre_e);
    ids_nn = load_ids(snn, 0);
    load_q(sn, qn);
    bt_base = 0;
    while (iss <= g_base + 2 && issuable()) issue_one();

    const int n_vis = row_ok ? sc.L - a.s_q + 1 + q_i : 0x7fffffff;
    f32x4 o[8];
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) o[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    for (int it = 0; it < sc.n; ++it) {
      const int ahead = iss - (g_base + it + 1);   // tiles issued after this one (<= 2)
      if (ahead >= 2) wait_vmcnt<2 * LPW>();
      else if (ahead == 1) wait_vmcnt<LPW>();
      else wait_vmcnt<0>();
      lds_barrier();   // tile it visible; every wave is done with tile it-1 and s_x
      // tile it+3 of the stream goes to the stage tile it-1 used; its copies
      // are spread over the score products below
      const bool do_iss = iss <= g_base + it + 3 && issuable();
      const uint8_t* isrc = a.kv;
      uint32_t idst = 0;
      if (do_iss) next_tile(isrc, idst);
      LDS_AS uint8_t* st = (LDS_AS uint8_t*)s_stage[(g_base + it) % NST];
      const int t0 = (sc.t_begin + it) * kTile;
      if (sc.L - t0 < kTile) clear_tail(st, sc.L - t0);

      // partial scores over this wave's k-steps, two 16-token blocks; all
      // operand reads first
      bf16x8 kf[2 * KQ];
#pragma unroll
      for (int j = 0; j < KQ; ++j) {
        if (j == KQ - 1 && !five) break;
        const int ks = ks0 + j;
        const LDS_AS uint8_t* kp = st + 4096 * (ks >> 1) + 512 * (ks & 1) + kofs;
        kf[2 * j] = lds_read_b128(kp);
        kf[2 * j + 1] = lds_read_b128(kp + 2048);
      }
      f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < KQ; ++j) {
        if (j == KQ - 1 && !five) break;
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[2 * j], qf[j], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[2 * j + 1], qf[j], acc1, 0, 0, 0);
        if (j < 4 && do_iss) {
          dma16_sbase_nt(isrc + 256 * j, doff, idst + 8192 * j);
          dma16_sbase_nt(isrc + 256 * j + 128, doff, idst + 8192 * j + 4096);
        }
      }
      if (do_iss) dma16_sbase_nt(isrc + 128 * (LPW - 1), doff, idst + 4096 * (LPW - 1));
      s_x[wave][0][lane] = acc0;
      s_x[wave][1][lane] = acc1;
      lds_barrier();   // partials visible (and the cleared tail)
      // value operands of the tile, in flight while the softmax runs
      bf16x8 vf[8];
#pragma unroll
      for (int ct = 0; ct < 8; ++ct)
        vf[ct] = vt_fragment(st + vb[0] + 4096 * (ct >> 2) + 256 * (ct & 3),
                             st + vb[1] + 4096 * (ct >> 2) + 256 * (ct & 3));
      // the four partials as (p[w] + p[w^1]) + (p[w^2] + p[w^3]), this wave's
      // own from registers: addition commutes, so every wave forms the same
      // pairs and holds the same sums
      const f32x4 sum0 = (acc0 + s_x[wave ^ 1][0][lane]) + (s_x[wave ^ 2][0][lane] + s_x[wave ^ 3][0][lane]);
      const f32x4 sum1 = (acc1 + s_x[wave ^ 1][1][lane]) + (s_x[wave ^ 2][1][lane] + s_x[wave ^ 3][1][lane]);

      // online softmax: element j of the lane is token 16 (j >> 2) + 4 g + (j & 3).
      // Interior tiles (every token visible to every row) skip the mask and
      // fold the scale into the exponent's FMA; masked tiles scale first and
      // then select, so that a masked token is -inf whatever the scale.
      const float c = a.scale_mag_log2;
      float alpha = 1.f;      // rescale factor of this lane's row (rare)
      bool rescale = false;   // some row's accumulators need it
      auto softmax = [&](auto masked_tag) {
        constexpr bool MASKED = decltype(masked_tag)::value;
        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float sj = j < 4 ? sum0[j] : sum1[j - 4];
          if (MASKED) {
            const int tok = t0 + 16 * (j >> 2) + 4 * g + (j & 3);
            x[j] = tok < n_vis ? sj * c : -INFINITY;
          } else {
            x[j] = sj;
          }
        }
        float lmax = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                           fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
        if (!MASKED) lmax *= c;
        if (__builtin_expect(__any(lmax > m_run + kRescaleThreshold), 0)) {
          // the four lanes of a row agree on its maximum
          float rmax = fmaxf(lmax, __shfl_xor(lmax, 16, 64));
          rmax = fmaxf(rmax, __shfl_xor(rmax, 32, 64));
          const bool raise = rmax > m_run + kRescaleThreshold;
          const float m_new = rmax + kRefHeadroom;
          alpha = raise ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
          rescale = __any(raise && m_run != -INFINITY);
          l_run *= alpha;
          if (raise) m_run = m_new;
        }
        const float neg_m = m_run == -INFINITY ? 0.f : -m_run;
        uint32_t pw[4];
        float psum = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p0 = __builtin_amdgcn_exp2f(MASKED ? x[2 * j] + neg_m
                                                         : __builtin_fmaf(x[2 * j], c, neg_m));
          const float p1 = __builtin_amdgcn_exp2f(MASKED ? x[2 * j + 1] + neg_m
                                                         : __builtin_fmaf(x[2 * j + 1], c, neg_m));
          psum += p0 + p1;
          pw[j] = pack_bf16x2(p0, p1);
        }
        l_run += psum;
        return __builtin_bit_cast(bf16x8, u32x4{pw[0], pw[1], pw[2], pw[3]});
      };
      const bf16x8 pb = __all(t0 + kTile <= n_vis) ? softmax(std::integral_constant<bool, false>{})
                                                   : softmax(std::integral_constant<bool, true>{});

      if (__builtin_expect(rescale, 0)) {
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) acc_scale4(o[ct], alpha);
      }

      // value product, output columns 128 wave + 16 ct + 4 g + (0..3) of row i16
#pragma unroll
      for (int ct = 0; ct < 8; ++ct)
        o[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[ct], pb, o[ct], 0, 0, 0);
    }

    // ---- epilogue: final rows, or bf16 partials of a split sequence
    float l_tot = l_run + __shfl_xor(l_run, 16, 64);
    l_tot += __shfl_xor(l_tot, 32, 64);
    const float inv_l = l_tot > 0.f ? 1.f / l_tot : 0.f;
    float lse_v = l_tot > 0.f ? (m_run + __log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
    if (bad_c) lse_v = __builtin_nanf("");
    if (row_ok) {
      const int64_t row = (int64_t)b * a.M + r;
      uint16_t* dst = sc.split ? a.part_o + ((int64_t)sc.slot * a.M + r) * kDL : a.out + row * kDL;
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) {
        uint32_t w0, w1;
        if (bad_c) {
          w0 = w1 = 0x7FC07FC0u;
        } else {
          w0 = pack_bf16x2(o[ct][0] * inv_l, o[ct][1] * inv_l);
          w1 = pack_bf16x2(o[ct][2] * inv_l, o[ct][3] * inv_l);
        }
        *reinterpret_cast<uint64_t*>(dst + 128 * wave + 16 * ct + 4 * g) =
            (uint64_t)w0 | ((uint64_t)w1 << 32);
      }
      if (wave == 0 && g == 0) {
        if (sc.split) a.part_lse[(int64_t)sc.slot * a.M + r] = lse_v;
        else a.lse[row] = lse_v;
      }
    }

    // Drain: the stores above, the prefetched tiles of the next segment, its
    // query rows and the id window after it. (Stores and loads may complete
    // out of order, so no partial count is exact after a store.)
    wait_vmcnt<0>();
    check_ids(snn, 0, ids_nn, bad_nn);
    g_base += sc.n;
    sc = sn;
    sn = snn;
    ids_c = ids_n;
    ids_n = ids_nn;
    bad_c = bad_n;
    bad_n = bad_nn;
    bad_nn = false;
  }
}

// Score-chain MFMA with its accumulator in VGPRs. With 256 AGPRs holding the
// value-product accumulators there is no AGPR room for the score tile, so it
// is pinned to VGPRs here (C/D of an MFMA may live in either file). `first`
// starts the chain from zero (literal srcC); the chain's own back-to-back
// SrcC dependency needs no wait states. mfma_vgpr_drain() must follow the
// last one before VALU code reads the result.
__device__ __forceinline__ void mfma_score(f32x16& acc, const bf16x8& a, const bf16x8& b, bool first) {
  if (first)   // early clobber: the result must not share registers with A or B
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
// The same with an A operand that VALU code has just written (an fp8 tile
// converted in registers): a VALU write of a VGPR that an MFMA then reads as
// SrcA/B needs 2 wait states, which the compiler does not insert ahead of
// an asm statement. `other` (the operand being converted for the next step)
// is held live across the MFMA, so that the conversions never write the
// registers an MFMA in flight is reading.
__device__ __forceinline__ void mfma_score_valu_a(f32x16& acc, const bf16x8& a, const bf16x8& b, bool first,
                                                  const bf16x8& other) {
  if (first)
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b), "v"(other));
  else
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b), "v"(other));
}
// The same chain on the fp8 matrix core: 32 tokens x 32 rows x 64 columns of
// E4M3 operands per instruction, 8 VGPRs (32 codes) of A and of B per lane.
// A lane's 32 codes are consecutive columns of one token (A) or one query
// row (B), taken by both operands in the same byte order, so the
// contraction is over the same 64 columns whatever order the matrix core
// sums them in. The E4M3 pairs are the default operand type (cbsz = blgp = 0).
__device__ __forceinline__ void mfma_score8(f32x16& acc, const u32x8& a, const u32x8& b, bool first) {
  if (first)
    asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
// XDL write (16 passes) -> VALU read of the same VGPRs
__device__ __forceinline__ void mfma8_vgpr_drain(f32x16& acc) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(acc));
}
// Query row value x (bf16, already in the score operand layout) as two E4M3
// codes with x * 2^e = hi + lo: hi = E4M3(x 2^e) rounded to nearest even and
// lo = E4M3(x 2^e - hi). x 2^e has at most 8 significant bits and hi takes the
// top 4 (rounded), so the remainder has at most 4 and is exact in E4M3 as
// long as it is a multiple of 2^-9 (|x 2^e| >= 1/4); with 2^e chosen per row
// so that the row's largest |x 2^e| lies in [128, 256), only values below
// 2^-9 of the row maximum lose bits of their lo part. Four bf16 (two words)
// in, one word of hi codes and one of lo codes out, byte i = value i.
// sd = 2^-e: the scaled conversions divide by their scale on the way to
// E4M3 and multiply by it on the way back, so hi comes straight from the
// bf16 pair and returns as hi 2^-e; h - x is one dot2 (x times -1 plus h,
// exact), converted with the same scale and its E4M3 sign bits flipped.
__device__ __forceinline__ void bf16x4_to_fp8_hilo(uint32_t w0, uint32_t w1, float sd, const DotSel& sel,
                                                    uint32_t& h, uint32_t& l) {
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  typedef short v2i16 __attribute__((ext_vector_type(2)));
  // hi through the builtins: their inputs come from lane swaps, whose
  // hazards the compiler resolves only for instructions it can see
  v2i16 hh = {0, 0};
  hh = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(hh, __builtin_bit_cast(bf16x2v, w0), sd, false);
  hh = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(hh, __builtin_bit_cast(bf16x2v, w1), sd, true);
  h = __builtin_bit_cast(uint32_t, hh);
  const auto b0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(h, sd, false);   // hi 2^-e, values 0, 1
  const auto b1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(h, sd, true);    // values 2, 3
  const bf16x2v x0 = __builtin_bit_cast(bf16x2v, w0), x1 = __builtin_bit_cast(bf16x2v, w1);
  const bf16x2v slo = __builtin_bit_cast(bf16x2v, sel.lo), shi = __builtin_bit_cast(bf16x2v, sel.hi);
  const float r0 = __builtin_amdgcn_fdot2_f32_bf16(x0, slo, b0[0], false);
  const float r1 = __builtin_amdgcn_fdot2_f32_bf16(x0, shi, b0[1], false);
  const float r2 = __builtin_amdgcn_fdot2_f32_bf16(x1, slo, b1[0], false);
  const float r3 = __builtin_amdgcn_fdot2_f32_bf16(x1, shi, b1[1], false);
  // lo in one asm block: its two halves are written by the two conversions,
  // so no prior contents are copied in. A scaled conversion needs a wait
  // state after the VALU write of a register it reads (the dot2 results, and
  // the second half-write reads the first's register), and its result one
  // before the next instruction reads it: the compiler cannot see into asm,
  // so the s_nops are written out
  uint32_t ll;
  asm("s_nop 1\n\t"
      "v_cvt_scalef32_pk_fp8_f32 %0, %1, %2, %5\n\t"
      "s_nop 0\n\t"
      "v_cvt_scalef32_pk_fp8_f32 %0, %3, %4, %5 op_sel:[0,0,0,1]\n\t"
      "s_nop 0"
      : "=&v"(ll) : "v"(r0), "v"(r1), "v"(r2), "v"(r3), "v"(sd));
  l = ll ^ 0x80808080u;
}
// max of three floats in one v_max3_f32; the asm also pins the result where
// it stands (no sinking into later conditional code).
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm volatile("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ void mfma_vgpr_drain(f32x16& acc) {
  // XDL write -> VALU read of the same VGPRs: more than 18 wait states
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(acc));
}

// --------------------------- bf16 decode kernel (128-row tile, pipelined)

// 128 query rows per workgroup, so every cache tile is streamed into exactly
// one CU (the LDS-DMA fill rate per CU is the scarce resource). Wave w:
//  * computes the full 576-column scores and the softmax of rows 32w..32w+31
//    (its query fragments stay in registers);
//  * publishes those rows' probabilities (bf16, already in the value
//    product's B-operand layout) through LDS;
//  * accumulates the value product of all 128 rows for output columns
//    128w..128w+127, so each V^T operand read from LDS feeds four MFMAs.
// Iteration i runs the dependent score chain of tile i (phase A, with the
// copies of tile i+2 and the first V reads of tile i-1 in its shadow), then
// the value product of tile i-1 with the online softmax of tile i cut into
// short VALU steps between its MFMAs (phase B). A 4-stage ring keeps tile
// i-1 resident while tile i is scored and tiles i+1, i+2 stream in. Over an
// fp8 (E4M3) cache the scores run on the fp8 matrix core against the query
// split once per sequence into two E4M3 parts (hi + lo under a power-of-two
// row scale, exact down to 2^-10 of the row maximum), the values on bf16
// MFMAs over codes converted exactly. The reference maximum of the online
// softmax moves rarely;
// when a row's does, its owner publishes the factor and every wave rescales
// that row's accumulators. The plan prefix and the epilogue's scratch live in
// ring space that is idle at those times, which keeps LDS under 160 KiB.
template <bool NT, bool FP8>
__global__ __launch_bounds__(256, 1) void mla_decode_pipe_kernel(DecodeParams a) {
  constexpr int NW = 4;
  constexpr int NTH = 64 * NW;
  constexpr int MT = 128;
  constexpr int NST = 4;                  // ring stages
  constexpr int LPW = 36 / NW;            // 1 KiB LDS-DMA loads per wave per tile (bf16)
  // score operands in flight (fp8: two 16-byte reads each)
  constexpr int KPF = FP8 ? 2 : 3;
  constexpr int KLG = FP8 ? 2 * KPF : KPF;   // LDS reads of those operands
  // fp8: the E4M3 tiles (18 KiB of codes + 128 B of scales) stream into
  // 19 KiB stages and are read as MFMA operands directly: the scores on the
  // fp8 matrix core against the query split into two E4M3 parts (hi + lo, one
  // power-of-two scale per row), the value product converted to bf16 in
  // registers (exact: every E4M3 value is a bf16 value); this halves the LDS
  // traffic of both products
  constexpr int STB = FP8 ? kFp8StageBytes : kTileBytes;   // bytes per ring stage
  // 4 x 36 KiB: the bf16 stages; the query rows pass through the upper half
  // (18 KiB a wave) before the third tile is issued, for both cache types
  constexpr int RING = 4 * kTileBytes;
  static_assert(NST * STB <= RING, "ring stages");
  using KOp = std::conditional_t<FP8, u32x8, bf16x8>;       // score operand as read
  // LDS-DMA copy of one block (NT: non-temporal, when no other workgroup
  // reads the same tiles)
  auto copy = [](const void* src, uint32_t off, uint32_t dst) {
    if constexpr (NT)
      dma16_sbase_nt(src, off, dst);
    else
      dma16_sbase(src, off, dst);
  };

  __shared__ __attribute__((aligned(1024))) uint8_t s_ring[RING];
  __shared__ __attribute__((aligned(16))) u32x4 s_p[NW][2][64];   // P, B-operand layout
  __shared__ float s_alpha[MT];
  __shared__ __attribute__((aligned(16))) int s_flag[NW];
  auto s_stage = [&](int i) { return s_ring + STB * i; };
  // aliases in the ring's last 36 KiB, which is idle before the first tile
  // and after the last one (fp8: never reached by the stages)
  uint8_t* const s_idle = s_ring + 3 * kTileBytes;
  int* s_pre = reinterpret_cast<int*>(s_idle);                    // [B+1]
  int* s_misc = reinterpret_cast<int*>(s_idle + 4 * (kMaxBatch + 8));
  float* s_lsum = reinterpret_cast<float*>(s_idle);               // epilogue

  const int tid = threadIdx.x, wave = uniform(tid >> 6);

  int v = blockIdx.x;
  const int G = gridDim.x;
  if ((G & 7) == 0) v = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
  const int part = v / a.m_tiles, mt = v % a.m_tiles;

  plan_prefix<NTH>(a.seqlens, a.B, a.max_blocks, s_pre, s_misc);
  const int T = uniform(s_pre[a.B]);
  const int P = a.P;
  if (blockIdx.x == 0)
    for (int b = tid; b <= a.B; b += NTH) a.ws_prefix[b] = s_pre[b];
  const int p_lo = part_start(part, P, T), p_hi = part_start(part + 1, P, T);
  int b_first, b_last;
  part_range<NTH>(s_pre, a.B, T, part == P - 1, p_lo, p_hi, s_misc, b_first, b_last);
  int pre_b = b_first <= b_last ? uniform(s_pre[b_first]) : 0;
  __syncthreads();   // ring stage 3 is free from here on

  const int cbase = 128 * wave;              // first output column of this wave

  for (int b = b_first; b <= b_last; ++b) {
    // Per-lane constants are derived here, from a lane index the compiler
    // cannot see through, so that they are not hoisted out of the sequence
    // loop and kept (spilled) across it.
    int tid_s = tid;
    asm volatile("" : "+v"(tid_s));
    const int lane = tid_s & 63, hi = lane >> 5, l32 = lane & 31;
    const int r = mt * MT + 32 * wave + l32;   // row whose scores this lane computes
    const bool row_ok = r < a.M;
    const int q_i = row_ok ? r / a.H : 0;
    // Score operand of k-step k (token l32, chunk 2k + hi): byte
    // 4096 (k >> 2) + 512 ((k >> 1) & 1) + (k odd ? kofs1 : kofs0).
    const int kR = l32 >> 3, kr = l32 & 7;
    const int kpart = 1024 * kR + 16 * ((kr & 3) | ((((kr >> 2) ^ hi) & 1) << 2) | (hi << 4));
    const int kofs0 = kpart + 128 * (kR & 1);
    const int kofs1 = kpart + 128 * ((kR & 1) ^ 1);
    // Value operand (transposing reads): lane (g16, i16) points at token
    // 4 vh + vs (+8 for the second read, +16 kk), chunk
    // 16 w + 4 cb + 2 (g16 & 1) + (vq >> 1), half vq & 1: byte
    // vofs{0,1} + 4096 (cb >> 1) + 512 (cb & 1) + 2048 kk.
    const int g16 = lane >> 4, i16 = lane & 15;
    const int vh = g16 >> 1, vq = i16 & 3, vs = i16 >> 2;
    const int vlane = 8192 * wave + 16 * vs + 64 * (vh ^ (vq >> 1)) + 256 * (vq >> 1) + 8 * (vq & 1);
    const int vofs0 = vlane + 128 * (g16 & 1);
    const int vofs1 = vlane + 1024 + 128 * ((g16 & 1) ^ 1);
    // LDS-DMA: copy j of wave w fills block 4 j + w (tokens 8w..8w+7, chunks
    // 8j..8j+7) from eight whole 128-byte lines; lane l's token and chunk
    // invert the in-block placement so that it lands at unit l.
    const int dc0 = (lane >> 4) & 1;
    const int dr = (lane & 3) | ((((lane >> 2) & 1) ^ dc0) << 2);
    const int dcc = dc0 | ((((lane >> 3) ^ wave) & 1) << 1) | (((lane >> 5) & 1) << 2);
    const uint32_t doff = (uint32_t)((8 * wave + dr) * kRowBytes + 16 * dcc);
    // fp8 stage: chunk k (16 codes, columns 16k..16k+15) of the 32 tokens
    // fills bytes 512 k .. 512 k + 511, token t in slot t ^ 4 (k & 1). A
    // score operand (8 codes of one token) is then one 8-byte read out of a
    // 512-byte run; the XOR puts the two chunks of a value read (transposing
    // read of 8 tokens x 16 columns per 16-lane group) in opposite halves of
    // the bank window. LDS-DMA copy m fills chunks 2m, 2m+1: lane l takes
    // chunk 2m + (l >> 5) of token (l & 31) ^ 4 (l >> 5).
    const uint32_t doff8 = (uint32_t)(kDK * ((lane & 31) ^ (4 * hi)) + 16 * hi);
    // fp8 score operand of k-step k (columns 64 k + 32 hi .. + 31 of token
    // l32): chunks 4 k + 2 hi (slot l32) and 4 k + 2 hi + 1 (slot l32 ^ 4),
    // byte 2048 k + kofs8_{0,1}
    const int kofs8_0 = 1024 * hi + 16 * l32;
    const int kofs8_1 = 1024 * hi + 512 + 16 * (l32 ^ 4);
    // value read: group g16 covers columns 16 (g16 & 1) + 0..15 of the column
    // block (chunk 8 w + 2 cb + (g16 & 1)); lane i16 = 2 s + h points at
    // codes 8h..8h+7 of the chunk for token 4 vh + (s & 3) + 8 (s >> 2) and
    // receives column i16 of those 8 tokens
    const int vs8 = i16 >> 1;
    const int vofs8 = 512 * (8 * wave + (g16 & 1)) +
                      16 * ((4 * vh + (vs8 & 3) + 8 * (vs8 >> 2)) ^ (4 * (g16 & 1))) + 8 * (i16 & 1);

    const int L = uniform(clamp_len(((const CONST_AS int32_t*)a.seqlens)[b], a.max_blocks));
    const int pre_e = pre_b + (L + kBT - 1) / kBT;
    const int seg_lo = max(p_lo, pre_b) - pre_b, seg_hi = min(p_hi, pre_e) - pre_b;
    bool split = false;
    int slot = 0;
    if (pre_e > pre_b) {
      const int fp = part_of(pre_b, P, T), lp = part_of(pre_e - 1, P, T);
      split = lp > fp;
      slot = 2 * part + ((part == fp && pre_b > p_lo) ? 1 : 0);
    }
    const int t_begin = 2 * seg_lo;
    const int t_end = min(2 * seg_hi, (L + kTile - 1) / kTile);
    const int n_tiles = max(0, t_end - t_begin);
    // an empty pool has no block to stand in for invalid ids: nothing is
    // streamed and the id check below poisons the segment
    const int n_run = a.num_blocks > 0 ? n_tiles : 0;
    const int n_vis = row_ok ? L - a.s_q + 1 + q_i : 0x7fffffff;

    f32x16 o[16];
    float zero = 0.f;
    asm volatile("" : "+v"(zero));   // no kernel-wide zero vector to keep alive
#pragma unroll
    for (int j = 0; j < 16; ++j)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[j][i] = zero;
    float m_run = -INFINITY, l_run = 0.f;

    // Block ids of the segment, 64 at a time, one per lane. Every wave loads
    // the same window, so the validity flag is uniform over the workgroup.
    // An id outside [0, num_blocks) poisons the segment (NaN output and lse)
    // and is replaced by block 0, so that no copy ever leaves the cache.
    const int seg_len = max(0, seg_hi - seg_lo);
    int bt_base = 0;
    int bt_lane = 0;
    bool bad = false;
    auto load_ids = [&]() {
      const int j = bt_base + min(lane, max(0, seg_len - bt_base - 1));
      bt_lane = seg_len > 0 ? ((const int32_t*)a.block_table)[(int64_t)b * a.max_blocks + seg_lo + j] : 0;
    };
    auto check_ids = [&]() {   // after the load has landed
      const bool inval = bt_lane < 0 || (int64_t)bt_lane >= a.num_blocks;
      bad = bad || __any(inval && bt_base + lane < seg_len);
      bt_lane = inval ? 0 : bt_lane;
    };
    // first cache row of tile idx (clamped to the segment's last tile)
    auto tile_row0 = [&](int idx) {
      idx = min(idx, n_run - 1);
      int rel = (idx >> 1) - bt_base;
      if (rel >= 64) {
        bt_base += 64;
        rel -= 64;
        load_ids();
        wait_vmcnt<0>();
        check_ids();
      }
      const int64_t phys = uniform(__builtin_amdgcn_readlane(bt_lane, rel));
      return phys * kBT + ((t_begin + idx) & 1) * kTile;
    };
    auto tile_src = [&](int idx) {
      if constexpr (FP8)
        return a.kv + tile_row0(idx) * kDK;
      else
        return a.kv + tile_row0(idx) * kRowBytes;
    };
    // fp8 copy j of this wave: copy m = wave + 4 j (m < 18: chunks 2m, 2m+1
    // of the tile's 32 rows, 32 bytes of each, the lines shared by copies
    // m..m+3 read from cache; m = 18: the tile's 128 bytes of scales, lanes
    // past them re-reading the first bytes into the stage's padding). Waves
    // 0..2 issue 5 copies per tile, wave 3 four.
    auto copy8 = [&](const uint8_t* src, const uint8_t* ssrc, uint32_t dst, int j) {
      const int m = wave + 4 * j;
      if (m < 18) {
        dma16_sbase(src + 32 * m, doff8, dst + 1024 * m);
      } else if (m == 18) {
        const int off = 16 * lane;
        dma16_sbase(ssrc, off < 4 * kTile ? off : 0, dst + kFp8TileBytes);
      }
    };
    auto issue = [&](int idx) {
      if constexpr (FP8) {
        const int64_t row0 = tile_row0(idx);
        const uint8_t* src = a.kv + row0 * kDK;
        const uint8_t* ssrc = a.kv_scales + row0 * 4;
        const uint32_t dst = lds_addr_of(s_stage(idx % NST));
#pragma unroll
        for (int j = 0; j < 5; ++j) copy8(src, ssrc, dst, j);
      } else {
        const uint32_t dst = lds_addr_of(s_stage(idx % NST)) + 1024 * wave;
        const uint8_t* src = tile_src(idx);
        // a tile past the last one is never used: its lanes all read one line
        const uint32_t d = idx < n_run ? doff : 0u;
#pragma unroll
        for (int j = 0; j < LPW; ++j) copy(src + 128 * j, d, dst + 4096 * j);
      }
    };
    // copies this wave issues per tile
    auto wait_tile = [&]() {
      if constexpr (FP8) {
        if (wave == 3)
          wait_vmcnt<4>();
        else
          wait_vmcnt<5>();
      } else {
        wait_vmcnt<LPW>();
      }
    };
    // fp8, last tile: codes and scales of the tokens past the end are zeroed
    // (they may hold anything, NaN included; the value product multiplies
    // them by zero probabilities)
    auto clear_tail8 = [&](LDS_AS uint8_t* st, int valid) {
      for (int u = tid; u < 36 * kTile; u += NTH) {
        const int token = (u & 31) ^ (4 * ((u >> 5) & 1));
        if (token >= valid) *reinterpret_cast<LDS_AS u32x4*>(st + 16 * u) = u32x4{0u, 0u, 0u, 0u};
      }
      if (tid < kTile && tid >= valid) reinterpret_cast<LDS_AS float*>(st + kFp8TileBytes)[tid] = 0.f;
    };
    auto clear_tail = [&](LDS_AS uint8_t* st, int valid) {   // bf16 only
      for (int u = tid; u < kTile * 72; u += NTH) {
        const int c0 = (u >> 4) & 1;
        const int token = 8 * ((u >> 6) & 3) + ((u & 3) | ((((u >> 2) & 1) ^ c0) << 2));
        if (token >= valid)
          *reinterpret_cast<LDS_AS f32x4*>(st + 16 * u) = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    };

    // The first block-id window and the query rows are loaded together; once
    // The block ids come first, alone, then the first two tiles are issued
    // into ring stages 0 and 1, and then the query rows, which pass through
    // ring stages 2 and 3 (idle until the third tile is issued), 18 KiB per
    // wave, to be read back in the score operand layout. (Issuing the query
    // rows together with the ids and the tiles once the ids had landed made
    // the ids wait behind the chip-wide burst of query loads: measured, the
    // prologue took about 1.4K cycles longer.)
    load_ids();
    bf16x8 qf[36];
    // fp8: the query rows as E4M3 hi and lo parts (score k-step k: columns
    // 64 k + 32 hi .. + 31 of row l32) and this row's score factor, the
    // softmax scale times 2^-e of the row's power-of-two scale
    u32x8 q8h[FP8 ? 9 : 1], q8l[FP8 ? 9 : 1];
    float c_row = a.scale_mag_log2;
    if (n_run > 0) {
      wait_vmcnt<0>();
      check_ids();
      issue(0);
      issue(1);
      // Query rows of this wave (32 rows, one contiguous 36 KiB block): load
      // 4 C + R takes block (C, R) of the K-tile layout (rows 8R..8R+7,
      // chunks 8C..8C+7) from eight whole 128-byte lines, each lane reading
      // the unit it holds in that block, the placement of the cache copies,
      // so that the LDS writes are contiguous and conflict-free. Rows past M
      // read row M-1 and are zeroed after the read.
      const uint8_t* qblk = reinterpret_cast<const uint8_t*>(a.q + (int64_t)b * a.M * kDK);
      const int row0 = mt * MT + 32 * wave;
      uint32_t qoff[4];
#pragma unroll
      for (int R = 0; R < 4; ++R) {
        const int dcq = dc0 | ((((lane >> 3) ^ R) & 1) << 1) | (((lane >> 5) & 1) << 2);
        qoff[R] = (uint32_t)(min(row0 + 8 * R + dr, a.M - 1) * kRowBytes + 16 * dcq);
      }
      u32x4 raw[36];
#pragma unroll
      for (int C = 0; C < 9; ++C)
#pragma unroll
        for (int R = 0; R < 4; ++R)
          raw[4 * C + R] = *reinterpret_cast<const u32x4*>(qblk + qoff[R] + 128 * C);
      asm volatile("" ::: "memory");
      // three passes of at most four column groups (16 KiB) each: write the
      // blocks, read back the k-steps they hold (a wave's LDS operations
      // complete in order, so a pass's writes follow the previous reads)
      LDS_AS uint8_t* stq = (LDS_AS uint8_t*)(s_ring + 2 * kTileBytes + (kTileBytes / 2) * wave);
      const uint32_t sg = row_ok ? a.q_sign2 : 0u;
      const uint32_t keep = row_ok ? 0xffffffffu : 0u;
#pragma unroll
      for (int pass = 0; pass < 3; ++pass) {
#pragma unroll
        for (int C = 4 * pass; C < 4 * pass + 4 && C < 9; ++C)
#pragma unroll
          for (int R = 0; R < 4; ++R)
            *reinterpret_cast<LDS_AS u32x4*>(stq + 1024 * (4 * (C - 4 * pass) + R) + 16 * lane) = raw[4 * C + R];
#pragma unroll
        for (int s2 = 16 * pass; s2 < 16 * pass + 16 && s2 < 36; ++s2) {
          const u32x4 z = __builtin_bit_cast(
              u32x4, lds_read_b128(stq + kstep_ofs(s2) - 16384 * pass + ((s2 & 1) ? kofs1 : kofs0)));
          qf[s2] = __builtin_bit_cast(bf16x8, (z ^ sg) & keep);
        }
      }
      if constexpr (FP8) {
        // row maximum of |x| (bf16 bits, NaN above every number) over the
        // lane's half of the row and its partner lane's
        u16x2 mx = {0, 0};
#pragma unroll
        for (int k = 0; k < 36; ++k) {
          const u32x4 w = __builtin_bit_cast(u32x4, qf[k]);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            mx = __builtin_elementwise_max(mx, __builtin_bit_cast(u16x2, w[i] & 0x7fff7fffu));
        }
        int m16 = max((int)mx[0], (int)mx[1]);
        m16 = max(m16, __shfl_xor(m16, 32, 64));
        // largest |x| 2^e in [128, 256); e clamped so that 2^e and 2^-e stay
        // normal fp32 (a row whose maximum is below 2^-93 or above 2^107 keeps
        // fewer exact bits in its small values)
        const int e = min(100, max(-100, 134 - ((m16 >> 7) & 0xff)));
        const float sd = __builtin_amdgcn_ldexpf(1.f, -e);
        c_row = a.scale_mag_log2 * sd;
        const DotSel sel;
        // lane (row, hi) holds chunks 2 k + hi of the row (8 columns each);
        // k-step k8 needs chunks 8 k8 + 4 hi + 0..3: swap halves with the
        // partner lane (the same row) before splitting
#pragma unroll
        for (int k8 = 0; k8 < 9; ++k8) {
          const u32x4 a0 = __builtin_bit_cast(u32x4, qf[4 * k8]);      // chunk 8k8 + hi
          const u32x4 a1 = __builtin_bit_cast(u32x4, qf[4 * k8 + 1]);  // 8k8 + 2 + hi
          const u32x4 b0 = __builtin_bit_cast(u32x4, qf[4 * k8 + 2]);  // 8k8 + 4 + hi
          const u32x4 b1 = __builtin_bit_cast(u32x4, qf[4 * k8 + 3]);  // 8k8 + 6 + hi
          u32x4 c[4];   // chunks 4 hi + 0..3
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const auto s0 = __builtin_amdgcn_permlane32_swap(a0[i], b0[i], false, false);
            const auto s1 = __builtin_amdgcn_permlane32_swap(a1[i], b1[i], false, false);
            c[0][i] = s0[0];
            c[1][i] = s0[1];
            c[2][i] = s1[0];
            c[3][i] = s1[1];
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            uint32_t h0, l0, h1, l1;
            bf16x4_to_fp8_hilo(c[j][0], c[j][1], sd, sel, h0, l0);
            bf16x4_to_fp8_hilo(c[j][2], c[j][3], sd, sel, h1, l1);
            q8h[k8][2 * j] = h0;
            q8h[k8][2 * j + 1] = h1;
            q8l[k8][2 * j] = l0;
            q8l[k8][2 * j + 1] = l1;
          }
        }
      }
      lds_barrier();   // every wave holds its query rows; stages 2 and 3 are free
      // "tile -1" (value product before the first tile) reads the last
      // stage with P = 0: both are zero-filled so that it adds exact zeros
      for (int u = tid; u < STB / 16; u += NTH)
        *reinterpret_cast<LDS_AS f32x4*>((LDS_AS uint8_t*)s_stage(NST - 1) + 16 * u) =
            f32x4{0.f, 0.f, 0.f, 0.f};
      s_p[wave][0][lane] = u32x4{0u, 0u, 0u, 0u};
      s_p[wave][1][lane] = u32x4{0u, 0u, 0u, 0u};
    } else {
      wait_vmcnt<0>();
      check_ids();
#pragma unroll
      for (int s = 0; s < 36; ++s) qf[s] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
      if constexpr (FP8) {
#pragma unroll
        for (int k8 = 0; k8 < 9; ++k8) {
#pragma unroll
          for (int i = 0; i < 8; ++i) q8h[k8][i] = q8l[k8][i] = 0u;
        }
      }
    }

    // Iteration it: scores and softmax of tile it (it < n_run), value product
    // of tile it-1 (it >= 1; "tile -1" adds zeros); tile it+2 streams in.
    // The first score operands of tile it are read at the end of iteration
    // it-1, before the barrier that publishes P(it-1), so that their LDS
    // latency is not exposed at the start of the score chain.
    KOp kf[KPF];
    auto rd_fp8 = [&](const LDS_AS uint8_t* st, int k) {
      const u32x4 c0 = __builtin_bit_cast(u32x4, lds_read_b128(st + 2048 * k + kofs8_0));
      const u32x4 c1 = __builtin_bit_cast(u32x4, lds_read_b128(st + 2048 * k + kofs8_1));
      return u32x8{c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
    };
    auto rd_at = [&](int t, int k) {
      const LDS_AS uint8_t* st = (const LDS_AS uint8_t*)s_stage(t % NST);
      if constexpr (FP8)
        return rd_fp8(st, k);
      else
        return lds_read_b128(st + kstep_ofs(k) + ((k & 1) ? kofs1 : kofs0));
    };
    if (n_run > 0) {
      wait_tile();                // tile 0 landed; tile 1 may be in flight
      lds_barrier();              // ... in every wave's part; the last stage and P zeroed
      if constexpr (FP8) {
        const int v0 = L - t_begin * kTile;
        if (v0 < kTile) {
          clear_tail8((LDS_AS uint8_t*)s_stage(0), v0);
          lds_barrier();
        }
      }
#pragma unroll
      for (int j2 = 0; j2 < KPF; ++j2) kf[j2] = rd_at(0, j2);
    }
    for (int it = 0; n_run > 0 && it <= n_run; ++it) {
      // P(it-1), alpha and flags of every wave are visible: their writes were
      // issued before the KPF score reads now in flight, and LDS operations
      // of a wave complete in order
      if (it > 0) asm volatile("s_waitcnt lgkmcnt(%0)\n\ts_barrier" ::"n"(KLG) : "memory");
      const bool has_s = it < n_run;
      const LDS_AS uint8_t* st = (const LDS_AS uint8_t*)s_stage(it % NST);
      const LDS_AS uint8_t* sp = (const LDS_AS uint8_t*)s_stage((it + NST - 1) % NST);
      const int t0 = (t_begin + it) * kTile;
      // rescale requests of tile it-1, read now and acted on after phase A
      const u32x4 flg = *reinterpret_cast<const u32x4*>(s_flag);
      const int64_t nrow0 = tile_row0(it + 2);
      const uint8_t* nsrc = a.kv + nrow0 * (FP8 ? kDK : kRowBytes);
      const uint8_t* nssrc = a.kv_scales + nrow0 * 4;   // fp8 only
      const uint32_t ndst = lds_addr_of(s_stage((it + 2) % NST)) + (FP8 ? 0 : 1024 * wave);
      // The loop's last two iterations copy a tile that is never used (the
      // copies stay in the code so that every iteration is the same); their
      // lanes all read the first 16 bytes of the clamped tile, one cache line
      // per instruction instead of eight.
      const uint32_t ndoff = it + 2 < n_run ? doff : 0u;

      // value step q = (kk, cb, rb) with kk = q / 16, cb = (q / 4) % 4,
      // rb = q % 4: O^T block (rb, cb) += V^T (column block cb, token half kk)
      // x P^T (rows of wave rb, token half kk)
      f32x16 s;
      auto rd = [&](int k) -> KOp {
        if constexpr (FP8)
          return rd_fp8(st, k);
        else
          return lds_read_b128(st + kstep_ofs(k) + ((k & 1) ? kofs1 : kofs0));
      };
      auto vread = [&](int kk, int cb) {
        if constexpr (FP8) {
          return vt_codes8(sp + vofs8 + 1024 * cb + 256 * kk);
        } else {
          const int o = 4096 * (cb >> 1) + 512 * (cb & 1) + 2048 * kk;
          return vt_fragment(sp + vofs0 + o, sp + vofs1 + o);
        }
      };
      // value operands, loaded in phase A's last third (fp8: va holds codes;
      // vb the current column block's operand, converted at the end of the
      // previous block)
      using VOp = std::conditional_t<FP8, u32x2, bf16x8>;
      bf16x8 pf[4], vb;
      VOp va[2];
      auto pv_step = [&](auto qc) {
        constexpr int q = decltype(qc)::value, cb = (q >> 2) & 3, rb = q & 3;
        if constexpr (FP8)
          o[4 * rb + cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vb, pf[rb], o[4 * rb + cb], 0, 0, 0);
        else
          o[4 * rb + cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[cb & 1], pf[rb], o[4 * rb + cb], 0, 0, 0);
        if constexpr (rb == 3 && q + 5 < 32) {
          // next V^T operand two column blocks ahead (token half changes at 16)
          constexpr int nq = q + 5;
          va[cb & 1] = vread(nq >> 4, (nq >> 2) & 3);
        }
        if constexpr (FP8) {
          if constexpr (rb == 3 && q + 1 < 32) vb = fp8x8_to_bf16(va[(cb + 1) & 1]);
        }
        // P^T of the second token half: each row block right after its last
        // use in the first half, four steps ahead of its first use
        if constexpr (q >= 12 && q < 16) pf[rb] = __builtin_bit_cast(bf16x8, s_p[rb][1][lane]);
      };
      // positions past the visible length (last tile, causal rows) score -inf;
      // in the last tile they may hold anything (their rows are zeroed only
      // after this tile's scores), the mask replaces whatever they score
      const bool masked = !__all(t0 + kTile <= n_vis);
      const int limx = masked ? n_vis - t0 - 4 * hi : kTile;
      __builtin_amdgcn_sched_barrier(0);

      // ---- phase A: the dependent score chain of tile it (36 bf16 MFMAs;
      // fp8: 18 fp8 MFMAs against the query's hi and lo parts) and the copy
      // of tile it+2; in its last third the first value operands of tile it-1
      // are read
      if constexpr (FP8) {
        // 9 k-steps of 64 columns, each operand read once and multiplied by
        // the hi and then the lo part of the query (one chain of 18 MFMAs)
        unroll<18>([&](auto jc) {
          constexpr int j = decltype(jc)::value, k = j >> 1;
          if constexpr (j & 1)
            mfma_score8(s, kf[k % KPF], q8l[k], false);
          else
            mfma_score8(s, kf[k % KPF], q8h[k], j == 0);
          if constexpr ((j & 1) && k + KPF < 9) kf[k % KPF] = rd(k + KPF);
          if constexpr (j >= 12 && j < 16) pf[j - 12] = __builtin_bit_cast(bf16x8, s_p[j - 12][0][lane]);
          if constexpr (j == 14) va[0] = vread(0, 0);
          if constexpr (j == 15) va[1] = vread(0, 1);
          if constexpr (j == 17) vb = fp8x8_to_bf16(va[0]);
          if constexpr ((j & 3) == 0) copy8(nsrc, nssrc, ndst, j >> 2);
          __builtin_amdgcn_sched_barrier(0);
        });
        mfma8_vgpr_drain(s);
      } else {
        unroll<36>([&](auto kc) {
          constexpr int k = decltype(kc)::value;
          mfma_score(s, kf[k % KPF], qf[k], k == 0);
          if constexpr (k + KPF < 36) kf[k % KPF] = rd(k + KPF);
          if constexpr (k >= 24 && k < 28) pf[k - 24] = __builtin_bit_cast(bf16x8, s_p[k - 24][0][lane]);
          if constexpr (k == 29) va[0] = vread(0, 0);
          if constexpr (k == 31) va[1] = vread(0, 1);
          if constexpr ((k & 3) == 1) copy(nsrc + 128 * (k >> 2), ndoff, ndst + 4096 * (k >> 2));
          __builtin_amdgcn_sched_barrier(0);
        });
        mfma_vgpr_drain(s);
      }

      // a row's reference maximum moved at tile it-1: rescale its
      // accumulators (which then hold tiles up to it-2) in every wave before
      // the value product of tile it-1 adds to them
      u32x4 flags = flg;
      asm volatile("" : "+v"(flags));   // keeps the read's wait out of phase A
      if (__builtin_expect((flags[0] | flags[1] | flags[2] | flags[3]) != 0 && it >= 2, 0)) {
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          if (flags[rb]) {           // only the row blocks whose maximum moved
            const float al = s_alpha[32 * rb + l32];
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) acc_scale(o[4 * rb + cb], al);
          }
        }
      }

      // ---- phase B: the value steps of tile it-1, with the online softmax of
      // tile it (own rows) cut into 28 short VALU steps between them (at most
      // about four VALU instructions and one exponential each, which is what
      // the shadow of one MFMA holds). It runs on every iteration and is
      // committed only when tile it exists; the empty asm statements keep each
      // step's results where the step stands, so that nothing is sunk into
      // the commit below. The row maximum pairs the two lane halves with a
      // lane swap; the reference maximum moves only when it is exceeded by
      // more than the threshold.
      const float c = FP8 ? c_row : a.scale_mag_log2;
      float x[16];
      f32x4 tsc4[4];   // fp8: per-token scales of the lane's tokens 8 g + 4 hi + (0..3)
      const LDS_AS float* tscp = reinterpret_cast<const LDS_AS float*>(st + kFp8TileBytes) + 4 * hi;
      float m01 = 0.f, m02 = 0.f, m03 = 0.f, m04 = 0.f, m05 = 0.f, m06 = 0.f, lmax = 0.f, rmax = 0.f;
      float m_new = m_run, alpha = 1.f, neg_m = 0.f, psum = 0.f, pprev = 0.f;
      bool raise = false;
      uint32_t pw[8];
      constexpr int NSM = 28;
      auto sm_step = [&](auto jc) {
        constexpr int st_ = decltype(jc)::value;
        if constexpr (st_ < 4) {
          if constexpr (FP8) {
            // tokens 8 st_ + 4 hi + (0..3); a token's score is scale * <q, row>
            const f32x4 v4 = *reinterpret_cast<const LDS_AS f32x4*>(tscp + 8 * st_);
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) x[4 * st_ + r4] = s[4 * st_ + r4] * (c * v4[r4]);
          } else {
#pragma unroll
            for (int i2 = 4 * st_; i2 < 4 * st_ + 4; ++i2) x[i2] = s[i2] * c;
          }
          if constexpr (st_ == 3) {
            if (masked) {
#pragma unroll
              for (int i2 = 0; i2 < 16; ++i2) x[i2] = 8 * (i2 >> 2) + (i2 & 3) < limx ? x[i2] : -INFINITY;
            }
          }
        } else if constexpr (st_ == 4) {
          m01 = max3f(x[0], x[1], x[2]);
          m02 = max3f(x[3], x[4], x[5]);
        } else if constexpr (st_ == 5) {
          m03 = max3f(x[6], x[7], x[8]);
          m04 = max3f(x[9], x[10], x[11]);
        } else if constexpr (st_ == 6) {
          m05 = max3f(x[12], x[13], x[14]);
          m06 = max3f(x[15], m01, m02);
        } else if constexpr (st_ == 7) {
          lmax = max3f(max3f(m03, m04, m05), m06, m06);
        } else if constexpr (st_ == 8) {
          const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lmax), __float_as_uint(lmax),
                                                           false, false);
          rmax = max3f(__uint_as_float(sw[0]), __uint_as_float(sw[1]), __uint_as_float(sw[1]));
        } else if constexpr (st_ == 9) {
          raise = rmax > m_run + kRescaleThreshold;
          m_new = raise ? rmax + kRefHeadroom : m_run;
          asm volatile("" : "+v"(m_new));
        } else if constexpr (st_ == 10) {
          if constexpr (FP8) tsc4[0] = *reinterpret_cast<const LDS_AS f32x4*>(tscp);
          alpha = raise ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
          asm volatile("" : "+v"(alpha));
        } else if constexpr (st_ == 11) {
          neg_m = m_new == -INFINITY ? 0.f : -m_new;
          asm volatile("" : "+v"(neg_m));
        } else {
          constexpr int j2 = st_ - 12;
          if constexpr (FP8 && (j2 & 3) == 2 && j2 + 2 < 16)   // scales of the next 4 tokens
            tsc4[(j2 + 2) >> 2] = *reinterpret_cast<const LDS_AS f32x4*>(tscp + 8 * ((j2 + 2) >> 2));
          const float p = __builtin_amdgcn_exp2f(x[j2] + neg_m);
          psum += p;
          if constexpr (j2 & 1) {
            // fp8: V is scale * value, the scale rides on the probability
            if constexpr (FP8)
              pw[j2 >> 1] = pack_bf16x2(pprev * tsc4[j2 >> 2][(j2 - 1) & 3], p * tsc4[j2 >> 2][j2 & 3]);
            else
              pw[j2 >> 1] = pack_bf16x2(pprev, p);
            asm volatile("" : "+v"(psum), "+v"(pw[j2 >> 1]));
          } else {
            pprev = p;
            asm volatile("" : "+v"(psum), "+v"(pprev));
          }
        }
      };
      constexpr int NB = 32;
      unroll<NB>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        pv_step(ic);
        unroll<NSM>([&](auto jc) {
          constexpr int j2 = decltype(jc)::value;
          if constexpr (1 + j2 == i) sm_step(jc);
        });
        __builtin_amdgcn_sched_barrier(0);
      });
      const bool raise_any = has_s && __any(raise);
      if (has_s) {
        l_run = l_run * alpha + psum;
        m_run = m_new;
        // last tile: zero rows past the end; its V serves the next iteration
        // (fp8: zeroed before its scores)
        if (!FP8 && L - t0 < kTile) clear_tail((LDS_AS uint8_t*)s_stage(it % NST), L - t0);
      }
      wait_tile();                // tile it+1 landed (this wave's part); tile it+2 in flight
      lds_barrier();              // every wave has read P(it-1) and tile it-1; tile it+1 visible
      if (has_s) {
        s_p[wave][0][lane] = u32x4{pw[0], pw[1], pw[2], pw[3]};
        s_p[wave][1][lane] = u32x4{pw[4], pw[5], pw[6], pw[7]};
        if (raise_any && hi == 0) s_alpha[32 * wave + l32] = alpha;
      }
      if (lane == 0) s_flag[wave] = raise_any ? 1 : 0;
      if constexpr (FP8) {
        // tile it+1 is the last: zero its tail before its scales are read
        // (the next barrier publishes it; a score read racing with it only
        // meets tokens that the mask drops)
        const int vn = L - (t0 + kTile);
        if (it + 1 < n_run && vn < kTile) clear_tail8((LDS_AS uint8_t*)s_stage((it + 1) % NST), vn);
      }
      asm volatile("" ::: "memory");   // the writes above are issued before the reads below
#pragma unroll
      for (int j2 = 0; j2 < KPF; ++j2) kf[j2] = rd_at(it + 1, j2);
    }

    // ---- epilogue (as in the 128-row kernel): rows staged through the idle
    // ring so that global stores are whole 256-byte row segments
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    float lse_v = l_tot > 0.f ? (m_run + __log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
    if (bad) lse_v = __builtin_nanf("");
    wait_vmcnt<0>();
    lds_barrier();
    if (hi == 0) s_lsum[32 * wave + l32] = l_tot;
    lds_barrier();
    constexpr int kStageRow = 272;
    uint16_t* dst_base = split ? a.part_o + ((int64_t)slot * a.M) * kDL
                               : a.out + ((int64_t)b * a.M) * kDL;
    LDS_AS uint8_t* stg = (LDS_AS uint8_t*)s_ring + wave * (64 * kStageRow);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int rb = 2 * half + q;
        const float lt = s_lsum[32 * rb + l32];
        const float inv_l = bad ? __builtin_nanf("") : (lt > 0.f ? 1.f / lt : 0.f);
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x16& acc = o[4 * rb + cb];
            const uint32_t w0 = pack_bf16x2(acc[4 * g + 0] * inv_l, acc[4 * g + 1] * inv_l);
            const uint32_t w1 = pack_bf16x2(acc[4 * g + 2] * inv_l, acc[4 * g + 3] * inv_l);
            const int col = 32 * cb + 8 * g + 4 * hi;
            *reinterpret_cast<LDS_AS uint64_t*>(stg + (32 * q + l32) * kStageRow + 2 * col) =
                (uint64_t)w0 | ((uint64_t)w1 << 32);
          }
      }
      lds_barrier();
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int rl0 = ln >> 4, cl = 8 * (ln & 15);
      const int row0 = mt * MT + 64 * half;
      uint16_t* gdst = dst_base + (int64_t)(row0 + rl0) * kDL + cbase + cl;
      const LDS_AS uint8_t* lsrc = stg + rl0 * kStageRow + 2 * cl;
      if (row0 + 64 <= a.M) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          *reinterpret_cast<u32x4*>(gdst + 4 * i * kDL) =
              *reinterpret_cast<const LDS_AS u32x4*>(lsrc + 4 * i * kStageRow);
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (row0 + rl0 + 4 * i < a.M)
            *reinterpret_cast<u32x4*>(gdst + 4 * i * kDL) =
                *reinterpret_cast<const LDS_AS u32x4*>(lsrc + 4 * i * kStageRow);
      }
      lds_barrier();
    }
    if (row_ok && hi == 0) {
      const int64_t row = (int64_t)b * a.M + r;
      if (!split)
        a.lse[row] = lse_v;
      else
        a.part_lse[(int64_t)slot * a.M + r] = lse_v;
    }
    wait_vmcnt<0>();
    __syncthreads();
    pre_b = pre_e;
  }
}

// ------------------ q8_0 / q4_0 decode kernel (128-row tile, converted tiles)

// Quantised cache (q8_0; with Q4 the q4_0 cache in Hadamard rotation), 128
// query rows per workgroup, 4 waves; wave w computes the scores and the
// softmax of rows 32w..32w+31 and the value product of all 128 rows for
// output columns 128w..128w+127 (the division of the 128-row bf16 kernel).
// Per 32-token tile, in four phases separated by barriers:
//  1. the int8 tile (18 KiB) and its scales (1152 B), copied by LDS-DMA into a
//     3-stage ring, are converted once by all threads into two bf16 tiles in
//     the row-group layout: hi = bf16(scale * value) and
//     lo = bf16(scale * value - hi). The product of an fp16 scale and an int8
//     value is exact in fp32 and hi + lo equals it to within 2^-17 relative,
//     so scores over hi and lo are the exact dequantised scores up to fp32
//     accumulation; tokens past the end of the sequence convert to zero;
//  2. scores S^T = K q~^T over hi and lo (two MFMA chains of 36 steps);
//  3. online softmax of the wave's rows (lazy reference maximum), P published
//     through LDS with the rescale requests;
//  4. value product O^T += V^T P^T with V = hi, the dequantised value rounded
//     to bf16.
// Compared with converting the int8 operands in every wave and scaling each
// 32-column group's partial score (the 32/64-row q8_0 kernel), the conversion
// work is done once per tile for all 128 rows and the scores are pure MFMA
// work.
// Q4: the q4_0 cache in Hadamard rotation (9 KiB of codes per tile). Step 1
// forms, per 32-column block, n = H (c - 8) on the matrix core (the integer
// Hadamard sums, exact), then x = d / sqrt(32) * n in fp32 and its hi / lo
// parts; everything after it is the q8_0 path.
template <bool NT, bool Q4 = false>
__global__ __launch_bounds__(256, 1) void mla_decode_q8w_kernel(DecodeParams a) {
  constexpr int NW = 4;
  constexpr int NTH = 64 * NW;
  constexpr int MT = 128;
  constexpr int NST = 3;                  // ring stages of the quantised tiles
  constexpr int KPF = 2;                  // score k-steps in flight (hi and lo each)
  // 1 KiB copies per wave per tile: q8_0 20 (5 a wave), q4_0 11 (3, wave 3 two)
  constexpr int NCOPY = Q4 ? 11 : 20;
  constexpr int CPW = (NCOPY + NW - 1) / NW;
  constexpr int CODE_COPIES = Q4 ? 9 : 18;
  constexpr int SCALE_OFF = Q4 ? kQ4TileBytes : kQ8TileBytes;   // scales in a stage
  constexpr int STAGE = Q4 ? kQ4StageBytes : kQ8StageBytes;

  __shared__ __attribute__((aligned(1024))) uint8_t s_ring[NST][STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t s_hl[2][kTileBytes];   // hi, lo
  __shared__ __attribute__((aligned(16))) u32x4 s_p[NW][2][64];   // P, B-operand layout
  __shared__ float s_alpha[MT];
  __shared__ __attribute__((aligned(16))) int s_flag[NW];
  // aliases inside the hi / lo tiles, which are idle before the first tile
  // and after the last one
  int* s_pre = reinterpret_cast<int*>(s_hl[0]);                   // [B+1]
  int* s_misc = reinterpret_cast<int*>(s_hl[1]);
  float* s_lsum = reinterpret_cast<float*>(s_hl[1] + 1024);       // epilogue
  static_assert(4 * (kMaxBatch + 1) <= kTileBytes, "plan prefix fits the hi tile");

  auto copy = [](const void* src, uint32_t off, uint32_t dst) {
    if constexpr (NT)
      dma16_sbase_nt(src, off, dst);
    else
      dma16_sbase(src, off, dst);
  };

  const int tid = threadIdx.x, wave = uniform(tid >> 6);

  int v = blockIdx.x;
  const int G = gridDim.x;
  if ((G & 7) == 0) v = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
  const int part = v / a.m_tiles, mt = v % a.m_tiles;

  plan_prefix<NTH>(a.seqlens, a.B, a.max_blocks, s_pre, s_misc);
  const int T = uniform(s_pre[a.B]);
  const int P = a.P;
  if (blockIdx.x == 0)
    for (int b = tid; b <= a.B; b += NTH) a.ws_prefix[b] = s_pre[b];
  const int p_lo = part_start(part, P, T), p_hi = part_start(part + 1, P, T);
  int b_first, b_last;
  part_range<NTH>(s_pre, a.B, T, part == P - 1, p_lo, p_hi, s_misc, b_first, b_last);
  int pre_b = b_first <= b_last ? uniform(s_pre[b_first]) : 0;
  __syncthreads();   // the hi / lo tiles are free from here on

  const int cbase = 128 * wave;              // first output column of this wave

  for (int b = b_first; b <= b_last; ++b) {
    // Per-lane constants are derived here, from a lane index the compiler
    // cannot see through, so that they are not hoisted out of the sequence
    // loop and kept (spilled) across it.
    int tid_s = tid;
    asm volatile("" : "+v"(tid_s));
    const int lane = tid_s & 63, hi = lane >> 5, l32 = lane & 31;
    const int r = mt * MT + 32 * wave + l32;   // row whose scores this lane computes
    const bool row_ok = r < a.M;
    const int q_i = row_ok ? r / a.H : 0;
    // Score operand of k-step k (token l32, chunk 2k + hi) in the row-group
    // layout: byte kstep_ofs(k) + (k odd ? kofs1 : kofs0).
    const int kR = l32 >> 3, kr = l32 & 7;
    const int kpart = 1024 * kR + 16 * ((kr & 3) | ((((kr >> 2) ^ hi) & 1) << 2) | (hi << 4));
    const int kofs0 = kpart + 128 * (kR & 1);
    const int kofs1 = kpart + 128 * ((kR & 1) ^ 1);
    // Value operand (transposing reads of the hi tile): lane (g16, i16)
    // points at token 4 vh + vs (+8 for the second read, +16 kk), chunk
    // 16 w + 4 cb + 2 (g16 & 1) + (vq >> 1), half vq & 1.
    const int g16 = lane >> 4, i16 = lane & 15;
    const int vh = g16 >> 1, vq = i16 & 3, vs = i16 >> 2;
    const int vlane = 64 * cbase + 16 * vs + 64 * (vh ^ (vq >> 1)) + 256 * (vq >> 1) + 8 * (vq & 1);
    const int vofs0 = vlane + 128 * (g16 & 1);
    const int vofs1 = vlane + 1024 + 128 * ((g16 & 1) ^ 1);

    const int L = uniform(clamp_len(((const CONST_AS int32_t*)a.seqlens)[b], a.max_blocks));
    const int pre_e = pre_b + (L + kBT - 1) / kBT;
    const int seg_lo = max(p_lo, pre_b) - pre_b, seg_hi = min(p_hi, pre_e) - pre_b;
    bool split = false;
    int slot = 0;
    if (pre_e > pre_b) {
      const int fp = part_of(pre_b, P, T), lp = part_of(pre_e - 1, P, T);
      split = lp > fp;
      slot = 2 * part + ((part == fp && pre_b > p_lo) ? 1 : 0);
    }
    const int t_begin = 2 * seg_lo;
    const int t_end = min(2 * seg_hi, (L + kTile - 1) / kTile);
    const int n_tiles = max(0, t_end - t_begin);
    // an empty pool has no block to stand in for invalid ids: nothing is
    // streamed and the id check below poisons the segment
    const int n_run = a.num_blocks > 0 ? n_tiles : 0;
    const int n_vis = row_ok ? L - a.s_q + 1 + q_i : 0x7fffffff;

    f32x16 o[16];
    float zero = 0.f;
    asm volatile("" : "+v"(zero));   // no kernel-wide zero vector to keep alive
#pragma unroll
    for (int j = 0; j < 16; ++j)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[j][i] = zero;
    float m_run = -INFINITY, l_run = 0.f;

    // Block ids of the segment, 64 at a time, one per lane (validated as in
    // the bf16 kernels: an id outside the pool poisons the segment and is
    // replaced by block 0).
    const int seg_len = max(0, seg_hi - seg_lo);
    int bt_base = 0;
    int bt_lane = 0;
    bool bad = false;
    auto load_ids = [&]() {
      const int j = bt_base + min(lane, max(0, seg_len - bt_base - 1));
      bt_lane = seg_len > 0 ? ((const int32_t*)a.block_table)[(int64_t)b * a.max_blocks + seg_lo + j] : 0;
    };
    auto check_ids = [&]() {   // after the load has landed
      const bool inval = bt_lane < 0 || (int64_t)bt_lane >= a.num_blocks;
      bad = bad || __any(inval && bt_base + lane < seg_len);
      bt_lane = inval ? 0 : bt_lane;
    };
    // Copies of int8 tile idx into ring stage idx % 3: copy k = wave + 4 j
    // (k < 18: bytes 1024 k .. of the tile's 32 rows, contiguous; k = 18, 19:
    // the 1152 bytes of scales, the tail of copy 19 reading the first bytes
    // again into the stage's padding).
    auto issue = [&](int idx) {
      int rel = (idx >> 1) - bt_base;   // lane of the segment's id window
      if (rel >= 64) {
        bt_base += 64;
        rel -= 64;
        load_ids();
        wait_vmcnt<0>();
        check_ids();
      }
      const int64_t phys = uniform(__builtin_amdgcn_readlane(bt_lane, rel));
      const int64_t row0 = phys * kBT + ((t_begin + idx) & 1) * kTile;
      const uint8_t* src = a.kv + row0 * (Q4 ? kQ4RowBytes : kQ8RowBytes);
      const uint32_t dst = lds_addr_of(s_ring[idx % NST]);
      const uint8_t* ssrc = a.kv_scales + row0 * kQ8ScaleRowBytes;
#pragma unroll
      for (int j = 0; j < CPW; ++j) {
        const int k = wave + 4 * j;
        if (k < CODE_COPIES) {
          copy(src + 1024 * k, 16 * lane, dst + 1024 * k);
        } else if (k < NCOPY) {
          // scales: default policy (the tail lanes re-read a partial line)
          const int off = 1024 * (k - CODE_COPIES) + 16 * lane;
          dma16_sbase(ssrc, off < kQ8ScaleTileBytes ? off : 0,
                      dst + SCALE_OFF + 1024 * (k - CODE_COPIES));
        }
      }
    };
    // q4_0: A operand of the Hadamard product, H[m][k] for row m = l32 and
    // columns k = 8 hi + e (first MFMA) and 16 + 8 hi + e (second)
    bf16x8 hA0, hA1;
    if constexpr (Q4) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int k0 = 8 * hi + e;
        hA0[e] = (__bf16)((__builtin_popcount(l32 & k0) & 1) ? -1.f : 1.f);
        hA1[e] = (__bf16)((__builtin_popcount(l32 & (k0 + 16)) & 1) ? -1.f : 1.f);
      }
    }

    // Query fragments of this lane's row (B operand of the score MFMA): 16
    // bytes per k-step, read directly; rows past M read zero.
    load_ids();
    bf16x8 qf[36];
    {
      const uint8_t* qrow = reinterpret_cast<const uint8_t*>(a.q + ((int64_t)b * a.M + (row_ok ? r : 0)) * kDK);
      const uint32_t sg = row_ok ? a.q_sign2 : 0u;
      const uint32_t keep = row_ok ? 0xffffffffu : 0u;
#pragma unroll
      for (int s2 = 0; s2 < 36; ++s2) {
        const u32x4 z = *reinterpret_cast<const u32x4*>(qrow + 32 * s2 + 16 * hi);
        qf[s2] = __builtin_bit_cast(bf16x8, (z ^ sg) & keep);
      }
    }
    wait_vmcnt<0>();
    check_ids();
    if (n_run > 0) issue(0);
    if (n_run > 1) issue(1);

    for (int it = 0; it < n_run; ++it) {
      // ---- 1. int8 tile it landed (tile it+1 may be in flight); everyone is
      // done with the previous tile's hi / lo / P
      if (it + 1 < n_run) {
        if constexpr (NCOPY % NW == 0) {
          wait_vmcnt<CPW>();
        } else {
          if (wave < NCOPY % NW)
            wait_vmcnt<CPW>();
          else
            wait_vmcnt<CPW - 1>();
        }
      } else {
        wait_vmcnt<0>();
      }
      lds_barrier();
      if (it + 2 < n_run) issue(it + 2);
      if constexpr (Q4) {
        // Wave w converts blocks g = w, w + 4, w + 8, w + 12 and half of
        // block 16 or 17 (below): n = H (c - 8) by two MFMAs
        // (H rows against the codes as bf16(128 + c), bits 0x4300 | c, which
        // adds 4352 to row m = 0 only, taken off), then x = d / sqrt(32) * n
        // and its hi / lo parts. Lane (t, hi) holds n[m][t] for
        // m = 8 q + 4 hi + (0..3): bytes 8 hi .. 8 hi + 7 of chunk 4 g + q of
        // token t. Tokens past the end of the sequence get scale 0.
        const LDS_AS uint8_t* st = (const LDS_AS uint8_t*)s_ring[it % NST];
        const int valid = L - (t_begin + it) * kTile;
        const bool tok_ok = l32 < valid;
        auto nib8 = [](uint32_t w) {
          u32x4 r;
#pragma unroll
          for (int k = 0; k < 4; ++k)
            r[k] = ((w >> (8 * k)) & 0xFu) | (((w >> (8 * k + 4)) & 0xFu) << 16) | 0x43004300u;
          return __builtin_bit_cast(bf16x8, r);
        };
        LDS_AS uint8_t* hib = (LDS_AS uint8_t*)s_hl[0];
        LDS_AS uint8_t* lob = (LDS_AS uint8_t*)s_hl[1];
        // (the lo parts by lo_part: measured faster here, where each block is a
        // dependent chain, and slower in the q8_0 conversion below)
        const DotSel sel;
        // x = d / sqrt(32) * n for four consecutive rows m of one token, and
        // its hi / lo parts, to the 8 bytes at u of the two tiles
        auto put4 = [&](float dv, float n0, float n1, float n2, float n3, int u) {
          const float x0 = dv * n0, x1 = dv * n1, x2 = dv * n2, x3 = dv * n3;
          const uint32_t h0 = pack_bf16x2(x0, x1), h1 = pack_bf16x2(x2, x3);
          const uint32_t l0 = pack_bf16x2(lo_part(h0, x0, sel.lo), lo_part(h0, x1, sel.hi));
          const uint32_t l1 = pack_bf16x2(lo_part(h1, x2, sel.lo), lo_part(h1, x3, sel.hi));
          *reinterpret_cast<LDS_AS uint64_t*>(hib + u) = (uint64_t)h0 | ((uint64_t)h1 << 32);
          *reinterpret_cast<LDS_AS uint64_t*>(lob + u) = (uint64_t)l0 | ((uint64_t)l1 << 32);
        };
        // Blocks 0..15: wave w converts w, w + 4, w + 8, w + 12, reading the
        // codes and scale of the next one while the current one converts
        // (the last read is not used).
        auto rd_codes = [&](int g, uint32_t& w0, uint32_t& w1, uint16_t& sbits) {
          const LDS_AS uint8_t* cu = st + kQ4RowBytes * l32 + 16 * g;
          w0 = *reinterpret_cast<const LDS_AS uint32_t*>(cu + 4 * hi);
          w1 = *reinterpret_cast<const LDS_AS uint32_t*>(cu + 8 + 4 * hi);
          sbits = *reinterpret_cast<const LDS_AS uint16_t*>(st + SCALE_OFF + kQ8ScaleRowBytes * l32 + 2 * g);
        };
        uint32_t nw0, nw1;
        uint16_t nsb;
        rd_codes(wave, nw0, nw1, nsb);
        // the half block's codes and scale (below) are read now as well
        const int gh = 16 + (wave >> 1);
        const int th = 16 * (wave & 1) + (lane & 15), qd = lane >> 4;
        const uint32_t wh = *reinterpret_cast<const LDS_AS uint32_t*>(st + kQ4RowBytes * th + 16 * gh + 4 * qd);
        const uint16_t sbh = *reinterpret_cast<const LDS_AS uint16_t*>(st + SCALE_OFF + kQ8ScaleRowBytes * th + 2 * gh);
        for (int g = wave; g < 16; g += NW) {
          const uint32_t w0 = nw0, w1 = nw1;
          const uint16_t sbits = nsb;
          rd_codes(min(g + NW, 15), nw0, nw1, nsb);
          const float dv = tok_ok ? (float)__builtin_bit_cast(_Float16, sbits) * kInvSqrt32 : 0.f;
          const f32x16 zero4 = {};
          f32x16 n = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hA0, nib8(w0), zero4, 0, 0, 0);
          n = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hA1, nib8(w1), n, 0, 0, 0);
          if (hi == 0) n[0] -= 4352.f;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            put4(dv, n[4 * q], n[4 * q + 1], n[4 * q + 2], n[4 * q + 3],
                 16 * rg_unit(l32, 4 * g + q) + 8 * hi);
        }
        // Blocks 16 and 17, split by token halves so that every wave converts
        // four and a half blocks: wave w takes tokens 16 (w & 1) .. + 15 of
        // block 16 + (w >> 1) on 16x16x32 MFMAs. Lane l: token
        // th = 16 (w & 1) + (l & 15); A = H rows m = l & 15 (second MFMA
        // m + 16) at columns k = 8 (l >> 4) + e; B = codes k = 8 (l >> 4) + e
        // of token th (word l >> 4 of its 16 bytes); the results hold
        // n[m][th] for m = 4 (l >> 4) + (0..3) and m + 16.
        {
          // (the lane index is made opaque so that the H operands below are
          // formed here, not hoisted out of the tile loop and kept, spilled)
          int lx = lane;
          asm volatile("" : "+v"(lx));
          const int g = gh, l16 = lx & 15;
          // sign of H[m][k] = parity(m & k) = parity(l16 & 8 qd) ^ parity(l16 & e)
          // (^ (qd >> 1) for m + 16); bit e of byte r of the table is
          // parity(r & e)
          const uint32_t rmask = (uint32_t)(0x963C5AF066CCAA00ull >> (8 * (l16 & 7)));
          const uint32_t s0 = ((l16 >> 3) & qd & 1) ? 0x80008000u : 0u;
          const uint32_t s1 = (qd & 2) ? 0x80008000u : 0u;
          u32x4 ha, hb;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            ha[j] = 0x3F803F80u | (((rmask >> (2 * j)) & 1u) << 15) | (((rmask >> (2 * j + 1)) & 1u) << 31);
            ha[j] ^= s0;
            hb[j] = ha[j] ^ s1;
          }
          const bf16x8 a0 = __builtin_bit_cast(bf16x8, ha), a1 = __builtin_bit_cast(bf16x8, hb);
          const uint32_t w = wh;
          const float dv = th < valid ? (float)__builtin_bit_cast(_Float16, sbh) * kInvSqrt32 : 0.f;
          const f32x4 zero4 = {};
          f32x4 n0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, nib8(w), zero4, 0, 0, 0);
          const f32x4 n1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, nib8(w), zero4, 0, 0, 0);
          if (qd == 0) n0[0] -= 4352.f;
          // rows 4 qd .. 4 qd + 3 are half (qd & 1) of chunk 4 g + (qd >> 1)
          put4(dv, n0[0], n0[1], n0[2], n0[3], 16 * rg_unit(th, 4 * g + (qd >> 1)) + 8 * (qd & 1));
          put4(dv, n1[0], n1[1], n1[2], n1[3], 16 * rg_unit(th, 4 * g + 2 + (qd >> 1)) + 8 * (qd & 1));
        }
      } else {
        // Thread (w, l) converts unit 256 i + 64 w + l of the hi / lo tiles,
        // i = 0..8: token 8 w + r(l), chunk 8 i + c(l) (the row-group
        // placement inverted), i.e. one token per thread. All reads first,
        // then the arithmetic; tokens past the end of the sequence read as
        // zero.
        const LDS_AS uint8_t* st = (const LDS_AS uint8_t*)s_ring[it % NST];
        const int valid = L - (t_begin + it) * kTile;   // tokens of the tile in the sequence
        const int lane = tid & 63;
        const int c0 = (lane >> 4) & 1;
        const int rr = (lane & 3) | ((((lane >> 2) & 1) ^ c0) << 2);
        const int cc = c0 | ((((lane >> 3) ^ wave) & 1) << 1) | (((lane >> 5) & 1) << 2);
        const int t = 8 * wave + rr;
        const uint32_t keep = t < valid ? 0xffffffffu : 0u;
        const LDS_AS uint8_t* srow = st + kQ8RowBytes * t + 8 * cc;
        const LDS_AS uint32_t* scl =
            reinterpret_cast<const LDS_AS uint32_t*>(st + kQ8TileBytes + kQ8ScaleRowBytes * t);
        uint64_t raw[9];
        uint32_t sc2[9];
#pragma unroll
        for (int i = 0; i < 9; ++i) {
          raw[i] = *reinterpret_cast<const LDS_AS uint64_t*>(srow + 64 * i);
          sc2[i] = scl[i];   // scales of groups 2i, 2i+1; chunk 8i + cc is group 2i + (cc >> 2)
        }
        const int sh16 = 16 * (cc >> 2);
#pragma unroll
        for (int i = 0; i < 9; ++i) {
          // the scale is zeroed too: a NaN or infinite scale in an unused
          // slot would otherwise reach the value product as 0 * inf
          const float d = (float)__builtin_bit_cast(_Float16, (uint16_t)((sc2[i] & keep) >> sh16));
          const uint32_t wv[2] = {(uint32_t)raw[i] & keep, (uint32_t)(raw[i] >> 32) & keep};
          u32x4 whi, wlo;
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            const uint32_t word = wv[e2 >> 1];
            const float x0 = d * (float)(int8_t)(word >> (16 * (e2 & 1)));
            const float x1 = d * (float)(int8_t)(word >> (16 * (e2 & 1) + 8));
            const uint32_t h = pack_bf16x2(x0, x1);
            const float h0 = __builtin_bit_cast(float, h << 16);
            const float h1 = __builtin_bit_cast(float, h & 0xffff0000u);
            whi[e2] = h;
            wlo[e2] = pack_bf16x2(x0 - h0, x1 - h1);
          }
          const int U = tid + NTH * i;
          *reinterpret_cast<LDS_AS u32x4*>((LDS_AS uint8_t*)s_hl[0] + 16 * U) = whi;
          *reinterpret_cast<LDS_AS u32x4*>((LDS_AS uint8_t*)s_hl[1] + 16 * U) = wlo;
        }
      }
      lds_barrier();   // hi (and lo) of tile it visible

      // ---- 2. scores of the wave's 32 rows over hi and lo (two chains)
      const LDS_AS uint8_t* khi = (const LDS_AS uint8_t*)s_hl[0];
      const LDS_AS uint8_t* klo = (const LDS_AS uint8_t*)s_hl[1];
      auto rd = [&](const LDS_AS uint8_t* base, int k) {
        return lds_read_b128(base + kstep_ofs(k) + ((k & 1) ? kofs1 : kofs0));
      };
      f32x16 sh, sl;
      bf16x8 kh[KPF], kl[KPF];
#pragma unroll
      for (int j2 = 0; j2 < KPF; ++j2) {
        kh[j2] = rd(khi, j2);
        kl[j2] = rd(klo, j2);
      }
      __builtin_amdgcn_sched_barrier(0);
      unroll<36>([&](auto kc) {
        constexpr int k = decltype(kc)::value;
        mfma_score(sh, kh[k % KPF], qf[k], k == 0);
        mfma_score(sl, kl[k % KPF], qf[k], k == 0);
        if constexpr (k + KPF < 36) {
          kh[k % KPF] = rd(khi, k + KPF);
          kl[k % KPF] = rd(klo, k + KPF);
        }
        __builtin_amdgcn_sched_barrier(0);
      });
      mfma_vgpr_drain(sh);
      mfma_vgpr_drain(sl);

      // ---- 3. online softmax of the wave's rows (log2 domain); element i of
      // the lane is token 8 (i >> 2) + 4 hi + (i & 3) of row l32
      const int t0 = (t_begin + it) * kTile;
      const float cs = a.scale_mag_log2;
      const bool masked = !__all(t0 + kTile <= n_vis);
      const int limx = masked ? n_vis - t0 - 4 * hi : kTile;
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const bool vis = !masked || 8 * (i >> 2) + (i & 3) < limx;
        const float sv = (sh[i] + sl[i]) * cs;
        x[i] = vis ? sv : -INFINITY;
      }
      float lmax = max3f(x[0], x[1], x[2]);
      lmax = max3f(lmax, x[3], x[4]);
      lmax = max3f(lmax, x[5], x[6]);
      lmax = max3f(lmax, x[7], x[8]);
      lmax = max3f(lmax, x[9], x[10]);
      lmax = max3f(lmax, x[11], x[12]);
      lmax = max3f(lmax, x[13], x[14]);
      lmax = fmaxf(lmax, x[15]);
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lmax), __float_as_uint(lmax),
                                                       false, false);
      const float rmax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      const bool raise = rmax > m_run + kRescaleThreshold;
      const float m_new = raise ? rmax + kRefHeadroom : m_run;
      const float alpha = raise ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
      const float neg_m = m_new == -INFINITY ? 0.f : -m_new;
      float psum = 0.f;
      uint32_t pw[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float p0 = __builtin_amdgcn_exp2f(x[2 * j] + neg_m);
        const float p1 = __builtin_amdgcn_exp2f(x[2 * j + 1] + neg_m);
        psum += p0 + p1;
        pw[j] = pack_bf16x2(p0, p1);
      }
      l_run = l_run * alpha + psum;
      m_run = m_new;
      const bool raise_any = __any(raise);
      s_p[wave][0][lane] = u32x4{pw[0], pw[1], pw[2], pw[3]};
      s_p[wave][1][lane] = u32x4{pw[4], pw[5], pw[6], pw[7]};
      if (raise_any && hi == 0) s_alpha[32 * wave + l32] = alpha;
      if (lane == 0) s_flag[wave] = raise_any ? 1 : 0;
      lds_barrier();   // P, rescale factors and flags of every wave visible

      // ---- 4. value product: a row's accumulators are rescaled first when
      // its reference maximum moved (rare)
      const u32x4 flags = *reinterpret_cast<const u32x4*>(s_flag);
      if (__builtin_expect((flags[0] | flags[1] | flags[2] | flags[3]) != 0, 0)) {
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          if (flags[rb]) {
            const float al = s_alpha[32 * rb + l32];
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) acc_scale(o[4 * rb + cb], al);
          }
        }
      }
      // all value and probability operands are read before the MFMAs, so the
      // LDS latency is paid once
      const LDS_AS uint8_t* sv = (const LDS_AS uint8_t*)s_hl[0];
      bf16x8 pf[2][4], va[2][4];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          const int off = 4096 * (cb >> 1) + 512 * (cb & 1) + 2048 * kk;
          va[kk][cb] = vt_fragment(sv + vofs0 + off, sv + vofs1 + off);
        }
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) pf[kk][rb] = __builtin_bit_cast(bf16x8, s_p[rb][kk][lane]);
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int rb = 0; rb < 4; ++rb)
            o[4 * rb + cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[kk][cb], pf[kk][rb], o[4 * rb + cb], 0, 0, 0);
    }

    // ---- epilogue: rows staged through the idle hi / lo tiles so that global
    // stores are whole 256-byte row segments
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    float lse_v = l_tot > 0.f ? (m_run + __log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
    if (bad) lse_v = __builtin_nanf("");
    wait_vmcnt<0>();
    lds_barrier();
    if (hi == 0) s_lsum[32 * wave + l32] = l_tot;
    lds_barrier();
    constexpr int kStageRow = 272;
    uint16_t* dst_base = split ? a.part_o + ((int64_t)slot * a.M) * kDL
                               : a.out + ((int64_t)b * a.M) * kDL;
    LDS_AS uint8_t* stg = (LDS_AS uint8_t*)s_hl[0] + wave * (64 * kStageRow);
    static_assert(4 * 64 * kStageRow <= 2 * kTileBytes, "staging fits the hi / lo tiles");
    // the row sums are read before the staging area (which covers s_lsum) is
    // written
    float lt_row[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) lt_row[rb] = s_lsum[32 * rb + l32];
    lds_barrier();
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int rb = 2 * half + q;
        const float lt = lt_row[rb];
        const float inv_l = bad ? __builtin_nanf("") : (lt > 0.f ? 1.f / lt : 0.f);
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x16& acc = o[4 * rb + cb];
            const uint32_t w0 = pack_bf16x2(acc[4 * g + 0] * inv_l, acc[4 * g + 1] * inv_l);
            const uint32_t w1 = pack_bf16x2(acc[4 * g + 2] * inv_l, acc[4 * g + 3] * inv_l);
            const int col = 32 * cb + 8 * g + 4 * hi;
            *reinterpret_cast<LDS_AS uint64_t*>(stg + (32 * q + l32) * kStageRow + 2 * col) =
                (uint64_t)w0 | ((uint64_t)w1 << 32);
          }
      }
      lds_barrier();
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int rl0 = ln >> 4, cl = 8 * (ln & 15);
      const int row0 = mt * MT + 64 * half;
      uint16_t* gdst = dst_base + (int64_t)(row0 + rl0) * kDL + cbase + cl;
      const LDS_AS uint8_t* lsrc = stg + rl0 * kStageRow + 2 * cl;
      if (row0 + 64 <= a.M) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          *reinterpret_cast<u32x4*>(gdst + 4 * i * kDL) =
              *reinterpret_cast<const LDS_AS u32x4*>(lsrc + 4 * i * kStageRow);
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (row0 + rl0 + 4 * i < a.M)
            *reinterpret_cast<u32x4*>(gdst + 4 * i * kDL) =
                *reinterpret_cast<const LDS_AS u32x4*>(lsrc + 4 * i * kStageRow);
      }
      lds_barrier();
    }
    if (row_ok && hi == 0) {
      const int64_t row = (int64_t)b * a.M + r;
      if (!split)
        a.lse[row] = lse_v;
      else
        a.part_lse[(int64_t)slot * a.M + r] = lse_v;
    }
    wait_vmcnt<0>();
    __syncthreads();
    pre_b = pre_e;
  }
}

// ------------------------------------------------------------ combine

// Merge n (lse, O) parts of one row; one wave, 8 columns per lane.
template <typename PartPtr>
__device__ __forceinline__ void merge_row(int n, PartPtr part, uint16_t* out_row, float* lse_out) {
  const int lane = threadIdx.x & 63;
  float m = -INFINITY;
  bool has_nan = false;
  for (int s = 0; s < n; ++s) {
    const float l = *part.lse(s);
    has_nan |= isnan(l);
    m = fmaxf(m, l);
  }
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  float L;
  if (has_nan) {
    L = __builtin_nanf("");
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = __builtin_nanf("");
  } else if (m == -INFINITY) {
    L = -INFINITY;
  } else {
    float tot = 0.f;
    for (int s = 0; s < n; ++s) tot += expf(*part.lse(s) - m);
    L = m + logf(tot);
    for (int s = 0; s < n; ++s) {
      const float w = expf(*part.lse(s) - L);
      if (w == 0.f) continue;
      float x[8];
      part.o8(s, lane, x);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += w * x[e];
    }
  }
  uint16_t hb[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) hb[e] = f32_to_bf16_bits(acc[e]);
  uint4 pk;
  pk.x = hb[0] | ((uint32_t)hb[1] << 16);
  pk.y = hb[2] | ((uint32_t)hb[3] << 16);
  pk.z = hb[4] | ((uint32_t)hb[5] << 16);
  pk.w = hb[6] | ((uint32_t)hb[7] << 16);
  *reinterpret_cast<uint4*>(out_row + 8 * lane) = pk;
  if (lane == 0) *lse_out = L;
}

// Merge the parts of one split row (8 columns per lane). WPR = 1: one wave
// per row; WPR = 4 (sequences cut into many parts, few rows): the four waves
// of a workgroup share one row, each merging a quarter of its parts, and the
// four partial sums are added in LDS in a fixed order. Every wave loads every
// part's lse at once, one part per lane, and its first four parts' value rows
// in the same round trip (they are needed unless the row is poisoned or
// empty); later rows are read four at a time. Each row is weighted by
// w_s = exp(lse_s - L), L the merged lse.
template <int WPR>
__global__ __launch_bounds__(kThreads, 8) void mla_split_combine_kernel(DecodeParams a) {
  static_assert(WPR == 1 || WPR == 4, "waves per row");
  __shared__ float s_acc[WPR - 1 > 0 ? WPR - 1 : 1][8][64];
  const int b = blockIdx.x;
  const int wv = uniform(threadIdx.x >> 6);
  const int r = WPR == 1 ? blockIdx.y * 4 + wv : blockIdx.y;
  if (r >= a.M) return;   // uniform over the workgroup when WPR = 4
  const int pre_b = a.ws_prefix[b], pre_e = a.ws_prefix[b + 1], T = a.ws_prefix[a.B];
  if (pre_e <= pre_b) return;
  const int fp = part_of(pre_b, a.P, T), lp = part_of(pre_e - 1, a.P, T);
  if (lp == fp) return;
  const int n = lp - fp + 1;
  const int lane = threadIdx.x & 63;
  const bool first_shifted = pre_b > part_start(fp, a.P, T);
  auto slot = [&](int s) { return 2 * (fp + s) + ((s == 0 && first_shifted) ? 1 : 0); };
  auto o_row = [&](int s) {
    return *reinterpret_cast<const uint4*>(a.part_o + ((int64_t)slot(s) * a.M + r) * kDL + 8 * lane);
  };
  auto lse_of = [&](int s) { return a.part_lse[(int64_t)slot(s) * a.M + r]; };
  const int64_t row = (int64_t)b * a.M + r;
  uint16_t* out_row = a.out + row * kDL;
  constexpr float kLog2e = 1.4426950408889634f;
  constexpr int kRound = 4;
  const int lo = (wv % WPR) * n / WPR, hi = (wv % WPR + 1) * n / WPR;   // this wave's parts
  // The lse values first, so that waiting for them leaves the value rows in
  // flight. Both are read without branches (indexes clamped to the last part,
  // n >= 2 here): loads behind branches would make the compiler wait for all
  // of them at the join.
  const float lse_raw = lse_of(min(lane, n - 1));
  uint4 v[kRound];
#pragma unroll
  for (int j = 0; j < kRound; ++j) v[j] = o_row(min(lo + j, n - 1));
  const float lse0 = lane < n ? lse_raw : -INFINITY;   // parts 0..63
  // max (and NaN) over the parts' lse
  float m = lse0;
  bool has_nan = isnan(lse0);
  for (int s0 = 64; s0 < n; s0 += 64) {
    const int s = s0 + lane;
    const float l = s < n ? lse_of(s) : -INFINITY;
    has_nan |= isnan(l);
    m = fmaxf(m, l);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  has_nan = __any(has_nan);
  if (has_nan || m == -INFINITY) {
    if (wv % WPR != 0) return;
    const float fill = has_nan ? __builtin_nanf("") : 0.f;
    const uint32_t h = f32_to_bf16_bits(fill);
    const uint32_t w = h | (h << 16);
    *reinterpret_cast<uint4*>(out_row + 8 * lane) = uint4{w, w, w, w};
    if (lane == 0) a.lse[row] = has_nan ? __builtin_nanf("") : -INFINITY;
    return;
  }
  // merged lse
  float tot = lane < n ? __builtin_amdgcn_exp2f((lse0 - m) * kLog2e) : 0.f;
  for (int s0 = 64; s0 < n; s0 += 64) {
    const int s = s0 + lane;
    if (s < n) tot += __builtin_amdgcn_exp2f((lse_of(s) - m) * kLog2e);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) tot += __shfl_xor(tot, off, 64);
  const float L = m + __log2f(tot) * 0.69314718055994531f;
  // weights of parts 0..63, part i in lane i; later parts' weights are
  // computed when they are used
  const float wl0 = lane < n ? __builtin_amdgcn_exp2f((lse0 - L) * kLog2e) : 0.f;
  auto weight_of = [&](int s) {
    if (s < 64) return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl0), s));
    return __builtin_amdgcn_exp2f((lse_of(s) - L) * kLog2e);
  };
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  for (int c0 = lo; c0 < hi; c0 += kRound) {
    if (c0 != lo) {
#pragma unroll
      for (int j = 0; j < kRound; ++j) v[j] = o_row(min(c0 + j, n - 1));
    }
#pragma unroll
    for (int j = 0; j < kRound; ++j) {
      if (c0 + j < hi) {
        const float w = weight_of(c0 + j);
        const uint32_t u[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] += w * __builtin_bit_cast(float, u[e] << 16);
          acc[2 * e + 1] += w * __builtin_bit_cast(float, u[e] & 0xffff0000u);
        }
      }
    }
  }
  if constexpr (WPR > 1) {
    if (wv > 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) s_acc[wv - 1][e][lane] = acc[e];
    }
    __syncthreads();
    if (wv > 0) return;
#pragma unroll
    for (int k = 0; k < WPR - 1; ++k)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += s_acc[k][e][lane];
  }
  uint4 pk;
  pk.x = f32_to_bf16_bits(acc[0]) | ((uint32_t)f32_to_bf16_bits(acc[1]) << 16);
  pk.y = f32_to_bf16_bits(acc[2]) | ((uint32_t)f32_to_bf16_bits(acc[3]) << 16);
  pk.z = f32_to_bf16_bits(acc[4]) | ((uint32_t)f32_to_bf16_bits(acc[5]) << 16);
  pk.w = f32_to_bf16_bits(acc[6]) | ((uint32_t)f32_to_bf16_bits(acc[7]) << 16);
  *reinterpret_cast<uint4*>(out_row + 8 * lane) = pk;
  if (lane == 0) a.lse[row] = L;
}

struct DenseParts {   // caller-provided partials [S, R, 512] / [S, R]
  const float* part_o;
  const float* part_lse;
  int64_t R, r;
  __device__ const float* lse(int s) const { return part_lse + (int64_t)s * R + r; }
  __device__ void o8(int s, int lane, float x[8]) const {
    const float4* src = reinterpret_cast<const float4*>(part_o + ((int64_t)s * R + r) * kDL + 8 * lane);
    const float4 x0 = src[0], x1 = src[1];
    x[0] = x0.x; x[1] = x0.y; x[2] = x0.z; x[3] = x0.w;
    x[4] = x1.x; x[5] = x1.y; x[6] = x1.z; x[7] = x1.w;
  }
};

__global__ __launch_bounds__(kThreads) void mla_combine_kernel(int S, int64_t R,
                                                               const float* part_o,
                                                               const float* part_lse,
                                                               uint16_t* out, float* lse) {
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= R) return;
  DenseParts parts{part_o, part_lse, R, r};
  merge_row(S, parts, out + r * kDL, lse + r);
}

// ------------------------------------------------------------ plan export

__global__ __launch_bounds__(kThreads) void mla_plan_kernel(const int32_t* seqlens, int B,
                                                            int max_blocks, int P,
                                                            int32_t* plan) {
  __shared__ int pre[kMaxBatch + 1];
  __shared__ int wsum[16];
  plan_prefix<kThreads>(seqlens, B, max_blocks, pre, wsum);
  const int T = pre[B];
  int32_t* o_pre = plan;
  int32_t* o_ps = o_pre + B + 1;
  int32_t* o_fp = o_ps + P + 1;
  int32_t* o_lp = o_fp + B;
  for (int b = threadIdx.x; b <= B; b += kThreads) o_pre[b] = pre[b];
  for (int p = threadIdx.x; p <= P; p += kThreads) o_ps[p] = part_start(p, P, T);
  for (int b = threadIdx.x; b < B; b += kThreads) {
    const int lo = pre[b], hi = pre[b + 1];
    if (hi > lo) {
      o_fp[b] = part_of(lo, P, T);
      o_lp[b] = part_of(hi - 1, P, T);
    } else {
      const int owner = lo < T ? part_of(lo, P, T) : P - 1;
      o_fp[b] = owner;
      o_lp[b] = owner;
    }
  }
}

// ================================================================== host

thread_local std::string g_last_error;

mla_status fail(mla_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
mla_status fail(mla_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

mla_status ok() {
  g_last_error.clear();
  return MLA_OK;
}

}  // namespace

namespace mla_internal {
// error string of the other entry points of the library (csrc/mla_proj.hip)
__attribute__((visibility("hidden"))) void set_last_error(const char* msg) { g_last_error = msg; }
}  // namespace mla_internal

namespace {

int device_cus() {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return -1;
  std::lock_guard<std::mutex> lock(mu);
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      return -1;
    cache[dev] = n;
  }
  return cache[dev];
}

struct Plan {
  bool narrow;   // 16-row tile (bf16 cache)
  bool q8w;      // q8_0 or q4_0 cache, 128-row tile converted to bf16 in LDS
  int HG, CG, MT, m_tiles, P, M;
  size_t off_prefix, off_lse, off_o, bytes;
};

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

mla_status validate_problem(const mla_problem* p) {
  if (!p) return fail(MLA_ERR_INVALID_ARG, "problem descriptor is NULL");
  if (p->batch < 0) return fail(MLA_ERR_INVALID_ARG, "batch must be >= 0 (got %d)", p->batch);
  if (p->batch > MLA_MAX_BATCH)
    return fail(MLA_ERR_UNSUPPORTED, "batch %d exceeds %d", p->batch, MLA_MAX_BATCH);
  if (p->seqlen_q < 1) return fail(MLA_ERR_INVALID_ARG, "seqlen_q must be >= 1");
  if (p->num_heads < 1) return fail(MLA_ERR_INVALID_ARG, "num_heads must be >= 1");
  if ((int64_t)p->seqlen_q * p->num_heads > MLA_MAX_ROWS)
    return fail(MLA_ERR_UNSUPPORTED, "seqlen_q * num_heads exceeds %d", MLA_MAX_ROWS);
  if (p->max_blocks_per_seq < 1) return fail(MLA_ERR_INVALID_ARG, "max_blocks_per_seq must be >= 1");
  if ((int64_t)p->max_blocks_per_seq * MLA_BLOCK_TOKENS > INT32_MAX ||
      (int64_t)p->batch * p->max_blocks_per_seq > INT32_MAX / 2)
    return fail(MLA_ERR_UNSUPPORTED, "block table too large");
  if (p->num_blocks < 0) return fail(MLA_ERR_INVALID_ARG, "num_blocks must be >= 0");
  if (p->max_seqlen < 0) return fail(MLA_ERR_INVALID_ARG, "max_seqlen must be >= 0");
  if (p->kv_dtype != MLA_KV_BF16 && p->kv_dtype != MLA_KV_Q8_0 && p->kv_dtype != MLA_KV_FP8 &&
      p->kv_dtype != MLA_KV_Q4_0H)
    return fail(MLA_ERR_INVALID_ARG, "unknown kv_dtype %d", p->kv_dtype);
  if (p->num_parts < 0) return fail(MLA_ERR_INVALID_ARG, "num_parts must be >= 0");
  if (p->m_tile != 0 && p->m_tile != 16 && p->m_tile != 32 && p->m_tile != 64 &&
      p->m_tile != 128)
    return fail(MLA_ERR_INVALID_ARG, "m_tile must be 0, 16, 32, 64 or 128 (got %d)", p->m_tile);
  return MLA_OK;
}

// Work split: HG row groups per workgroup from the rows per sequence, and P
// partitions so that P * m_tiles workgroups about fill the compute units.
mla_status make_plan(const mla_problem* p, Plan* pl) {
  mla_status s = validate_problem(p);
  if (s != MLA_OK) return s;
  const int M = p->seqlen_q * p->num_heads;
  pl->M = M;
  // Row tile. bf16 cache: 16 rows per workgroup (the four waves split the
  // score contraction and the output columns), or 32, 64 or 128 (1, 2 or 4
  // row groups of 32, each wave owning whole rows); the smallest tile that
  // holds all rows of a sequence, so the cache is streamed once per part.
  // q8_0 cache: 32 or 64 rows, each row group's work split over 4 waves, or
  // 128 rows (the tile converted once into exact bf16 hi / lo parts). fp8
  // cache: 128 rows (the bf16 pipeline, its operands read as E4M3 codes and
  // converted exactly in registers). q4_0 cache in Hadamard rotation: as
  // q8_0 (its 128-row tile converted through the matrix core). More rows
  // than one tile holds take
  // several row tiles per KV part, placed on the same XCD so the second read
  // of each cache tile hits L2.
  const bool q8 = p->kv_dtype == MLA_KV_Q8_0;
  const bool fp8 = p->kv_dtype == MLA_KV_FP8;
  const bool q4 = p->kv_dtype == MLA_KV_Q4_0H;
  if (q8 && p->m_tile == 16)
    return fail(MLA_ERR_UNSUPPORTED, "m_tile %d is not available for the q8_0 cache", p->m_tile);
  if (q4 && p->m_tile == 16)
    return fail(MLA_ERR_UNSUPPORTED, "m_tile %d is not available for the q4_0 cache", p->m_tile);
  if (fp8 && p->m_tile != 0 && p->m_tile != 128)
    return fail(MLA_ERR_UNSUPPORTED, "the fp8 cache takes 128-row tiles only (m_tile %d)",
                p->m_tile);
  pl->narrow = !q8 && !fp8 && !q4 && (p->m_tile == 16 || (p->m_tile == 0 && M <= 16));
  if (pl->narrow) {
    pl->HG = 1;
  } else if (fp8) {
    pl->HG = 4;
  } else if (p->m_tile) {
    pl->HG = p->m_tile / 32;
  } else {
    pl->HG = M <= 32 ? 1 : (M <= 64 ? 2 : 4);
  }
  pl->q8w = (q8 || q4) && pl->HG == 4;
  pl->CG = (q8 || q4) ? (pl->q8w ? 1 : 4) : 4 / pl->HG;
  pl->MT = pl->narrow ? 16 : 32 * pl->HG;
  pl->m_tiles = (M + pl->MT - 1) / pl->MT;
  int P = p->num_parts;
  if (P == 0) {
    const int cus = device_cus();
    if (cus <= 0) return fail(MLA_ERR_HIP, "cannot query the device's compute-unit count");
    const int64_t cap_tokens =
        (int64_t)p->max_blocks_per_seq * MLA_BLOCK_TOKENS;
    const int64_t ms = p->max_seqlen > 0 ? (p->max_seqlen < cap_tokens ? p->max_seqlen : cap_tokens)
                                         : cap_tokens;
    const int64_t t_max = (int64_t)p->batch * ((ms + MLA_BLOCK_TOKENS - 1) / MLA_BLOCK_TOKENS);
    // one workgroup per CU; when the cache has fewer blocks than that, parts
    // of a single block (two tiles) still cut the latency of small problems,
    // since all parts run at once and their merge is short
    int64_t want = cus / pl->m_tiles;
    if (want > t_max) want = t_max;
    if (want < 1) want = 1;
    P = (int)want;
  }
  if ((int64_t)P * pl->m_tiles > INT32_MAX / 2) return fail(MLA_ERR_UNSUPPORTED, "too many parts");
  pl->P = P;
  size_t off = 0;
  pl->off_prefix = off;
  off = align_up(off + 4 * ((size_t)p->batch + 1), 256);
  pl->off_lse = off;
  if (P > 1) {
    off = align_up(off + (size_t)2 * P * M * 4, 256);
    pl->off_o = off;
    off += (size_t)2 * P * M * kDL * 2;   // bf16 partials
  } else {
    pl->off_o = off;
  }
  pl->bytes = off;
  return MLA_OK;
}

bool aligned(const void* ptr, size_t a) { return ((uintptr_t)ptr % a) == 0; }

template <int HG, int CG, bool Q8, bool Q4 = false>
hipError_t launch_decode(const DecodeParams& dp, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((mla_decode_kernel<HG, CG, Q8, Q4>), dim3(grid), dim3(64 * HG * CG), 0,
                     stream, dp);
  return hipGetLastError();
}

template <bool FP8>
hipError_t launch_pipe(const DecodeParams& dp, int grid, hipStream_t stream) {
  if (dp.m_tiles == 1)
    hipLaunchKernelGGL((mla_decode_pipe_kernel<true, FP8>), dim3(grid), dim3(256), 0, stream, dp);
  else
    hipLaunchKernelGGL((mla_decode_pipe_kernel<false, FP8>), dim3(grid), dim3(256), 0, stream, dp);
  return hipGetLastError();
}

template <bool Q4>
hipError_t launch_q8w(const DecodeParams& dp, int grid, hipStream_t stream) {
  if (dp.m_tiles == 1)
    hipLaunchKernelGGL((mla_decode_q8w_kernel<true, Q4>), dim3(grid), dim3(256), 0, stream, dp);
  else
    hipLaunchKernelGGL((mla_decode_q8w_kernel<false, Q4>), dim3(grid), dim3(256), 0, stream, dp);
  return hipGetLastError();
}

hipError_t launch_narrow(const DecodeParams& dp, int grid, hipStream_t stream) {
  hipLaunchKernelGGL(mla_decode_narrow_kernel, dim3(grid), dim3(256), 0, stream, dp);
  return hipGetLastError();
}

template <int HG>
hipError_t launch_rows(const DecodeParams& dp, int grid, hipStream_t stream) {
  if (dp.m_tiles == 1)
    hipLaunchKernelGGL((mla_decode_rows_kernel<HG, true>), dim3(grid), dim3(256), 0, stream, dp);
  else
    hipLaunchKernelGGL((mla_decode_rows_kernel<HG, false>), dim3(grid), dim3(256), 0, stream, dp);
  return hipGetLastError();
}

// Host-side checks shared by the decode entry points; fills *pl.
mla_status check_decode_args(const mla_problem* p, const void* q, const void* kv_cache,
                             const void* kv_scales, const int32_t* block_table,
                             const int32_t* seqlens, float softmax_scale, const void* out,
                             const float* lse, Plan* pl) {
  mla_status s = validate_problem(p);
  if (s != MLA_OK) return s;
  if (p->batch == 0) return ok();
  if (!q || !kv_cache || !block_table || !seqlens || !out || !lse)
    return fail(MLA_ERR_INVALID_ARG, "null array argument");
  if (p->kv_dtype != MLA_KV_BF16 && !kv_scales)
    return fail(MLA_ERR_INVALID_ARG, "kv_scales is required for a quantised cache");
  if (!aligned(q, 16) || !aligned(kv_cache, 16) || !aligned(out, 16))
    return fail(MLA_ERR_INVALID_ARG, "q, kv_cache and out must be 16-byte aligned");
  if (!aligned(lse, 4) || !aligned(block_table, 4) || !aligned(seqlens, 4))
    return fail(MLA_ERR_INVALID_ARG, "lse, block_table and seqlens must be 4-byte aligned");
  if (p->kv_dtype != MLA_KV_BF16 && !aligned(kv_scales, 16))
    return fail(MLA_ERR_INVALID_ARG, "kv_scales must be 16-byte aligned");
  if (!(softmax_scale == softmax_scale) || isinf(softmax_scale))
    return fail(MLA_ERR_INVALID_ARG, "softmax_scale must be finite");
  return make_plan(p, pl);
}

mla_status launch_decode_step(const mla_problem* p, const Plan& pl, const void* q,
                              const void* kv_cache, const void* kv_scales,
                              const int32_t* block_table, const int32_t* seqlens,
                              float softmax_scale, void* out, float* lse, void* workspace,
                              hipStream_t stream);

// Workspace of mla_decode_noalloc: one array per device, held until the
// process ends. In host code `scratch` names a host-side stand-in, never the
// device memory: its device address is taken once per device with
// hipGetSymbolAddress and only that address is used.
constexpr size_t kScratchBytes = MLA_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

mla_status scratch_of_current_device(void** ptr) {
  static std::mutex mu;
  static void* addr[64] = {nullptr};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(MLA_ERR_UNSUPPORTED, "device index %d", dev);
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !a)
      return fail(MLA_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    addr[dev] = a;
  }
  *ptr = addr[dev];
  return MLA_OK;
}

}  // namespace

extern "C" {

const char* mla_status_str(mla_status s) {
  switch (s) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARG: return "MLA_ERR_INVALID_ARG";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED";
    case MLA_ERR_WORKSPACE_TOO_SMALL: return "MLA_ERR_WORKSPACE_TOO_SMALL";
    case MLA_ERR_HIP: return "MLA_ERR_HIP";
  }
  return "unknown mla_status";
}

const char* mla_last_error(void) { return g_last_error.c_str(); }

mla_status mla_workspace_size(const mla_problem* p, size_t* bytes) {
  if (!bytes) return fail(MLA_ERR_INVALID_ARG, "bytes is NULL");
  Plan pl;
  mla_status s = make_plan(p, &pl);
  if (s != MLA_OK) return s;
  *bytes = pl.bytes;
  return ok();
}

mla_status mla_num_parts(const mla_problem* p, int32_t* num_parts) {
  if (!num_parts) return fail(MLA_ERR_INVALID_ARG, "num_parts is NULL");
  Plan pl;
  mla_status s = make_plan(p, &pl);
  if (s != MLA_OK) return s;
  *num_parts = pl.P;
  return ok();
}

mla_status mla_decode(const mla_problem* p, const void* q, const void* kv_cache,
                      const void* kv_scales, const int32_t* block_table,
                      const int32_t* seqlens, float softmax_scale, void* out, float* lse,
                      void* workspace, size_t workspace_bytes, hipStream_t stream) {
  // everything checkable on the host, before any HIP call
  Plan pl;
  mla_status s = check_decode_args(p, q, kv_cache, kv_scales, block_table, seqlens,
                                   softmax_scale, out, lse, &pl);
  if (s != MLA_OK || p->batch == 0) return s;
  if (workspace && !aligned(workspace, 16))
    return fail(MLA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  if (workspace_bytes < pl.bytes)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu", pl.bytes,
                workspace_bytes);
  if (!workspace) return fail(MLA_ERR_INVALID_ARG, "workspace is NULL");
  return launch_decode_step(p, pl, q, kv_cache, kv_scales, block_table, seqlens, softmax_scale,
                            out, lse, workspace, stream);
}

mla_status mla_decode_noalloc(const mla_problem* p, const void* q, const void* kv_cache,
                              const void* kv_scales, const int32_t* block_table,
                              const int32_t* seqlens, float softmax_scale, void* out,
                              float* lse, hipStream_t stream) {
  Plan pl;
  mla_status s = check_decode_args(p, q, kv_cache, kv_scales, block_table, seqlens,
                                   softmax_scale, out, lse, &pl);
  if (s != MLA_OK || p->batch == 0) return s;
  if (pl.bytes > kScratchBytes)
    return fail(MLA_ERR_UNSUPPORTED,
                "this problem needs %zu bytes of workspace; mla_decode_noalloc holds at most "
                "%zu (MLA_NOALLOC_SCRATCH_BYTES): use mla_decode with a workspace",
                pl.bytes, (size_t)kScratchBytes);
  void* ws = nullptr;
  s = scratch_of_current_device(&ws);
  if (s != MLA_OK) return s;
  return launch_decode_step(p, pl, q, kv_cache, kv_scales, block_table, seqlens, softmax_scale,
                            out, lse, ws, stream);
}

}  // extern "C"

namespace {

mla_status launch_decode_step(const mla_problem* p, const Plan& pl, const void* q,
                              const void* kv_cache, const void* kv_scales,
                              const int32_t* block_table, const int32_t* seqlens,
                              float softmax_scale, void* out, float* lse, void* workspace,
                              hipStream_t stream) {
  DecodeParams dp;
  dp.q = (const uint16_t*)q;
  dp.kv = (const uint8_t*)kv_cache;
  dp.kv_scales = (const uint8_t*)kv_scales;
  dp.block_table = block_table;
  dp.seqlens = seqlens;
  dp.out = (uint16_t*)out;
  dp.lse = lse;
  uint8_t* ws = (uint8_t*)workspace;
  dp.ws_prefix = (int32_t*)(ws + pl.off_prefix);
  dp.part_lse = (float*)(ws + pl.off_lse);
  dp.part_o = (uint16_t*)(ws + pl.off_o);
  dp.num_blocks = p->num_blocks;
  dp.B = p->batch;
  dp.s_q = p->seqlen_q;
  dp.H = p->num_heads;
  dp.M = pl.M;
  dp.max_blocks = p->max_blocks_per_seq;
  dp.P = pl.P;
  dp.m_tiles = pl.m_tiles;
  // q4_0 in Hadamard rotation: the 32/64-row kernel's scores leave out the
  // rotation's 1 / sqrt(32), which is taken here (the 128-row kernel scales
  // its converted tile by it)
  const double rot = p->kv_dtype == MLA_KV_Q4_0H && !pl.q8w ? 0.17677669529663688110 : 1.0;
  dp.scale_log2 = (float)((double)softmax_scale * 1.4426950408889634074 * rot);
  dp.scale_mag_log2 = fabsf(dp.scale_log2);
  dp.q_sign2 = softmax_scale < 0.f ? 0x80008000u : 0u;

  const int grid = pl.P * pl.m_tiles;
  hipError_t e;
  // every cache type has its own kernels: a kernel reads the cache in its
  // own row size (1152 B bf16, 576 B int8 or E4M3, 288 B of q4_0 codes)
  switch (p->kv_dtype) {
    case MLA_KV_BF16:
      if (pl.narrow) {
        e = launch_narrow(dp, grid, stream);
      } else {
        switch (pl.HG) {
          case 1: e = launch_rows<1>(dp, grid, stream); break;
          case 2: e = launch_rows<2>(dp, grid, stream); break;
          case 4: e = launch_pipe<false>(dp, grid, stream); break;
          default: return fail(MLA_ERR_UNSUPPORTED, "no kernel for this row tile");
        }
      }
      break;
    case MLA_KV_Q8_0:
      if (pl.q8w)
        e = launch_q8w<false>(dp, grid, stream);
      else if (pl.HG == 2)
        e = launch_decode<2, 4, true>(dp, grid, stream);
      else if (pl.HG == 1)
        e = launch_decode<1, 4, true>(dp, grid, stream);
      else
        return fail(MLA_ERR_UNSUPPORTED, "no q8_0 kernel for this row tile");
      break;
    case MLA_KV_FP8:
      if (pl.HG != 4) return fail(MLA_ERR_UNSUPPORTED, "no fp8 kernel for this row tile");
      e = launch_pipe<true>(dp, grid, stream);
      break;
    case MLA_KV_Q4_0H:
      if (pl.q8w)
        e = launch_q8w<true>(dp, grid, stream);
      else if (pl.HG == 2)
        e = launch_decode<2, 4, true, true>(dp, grid, stream);
      else if (pl.HG == 1)
        e = launch_decode<1, 4, true, true>(dp, grid, stream);
      else
        return fail(MLA_ERR_UNSUPPORTED, "no q4_0 kernel for this row tile");
      break;
    default:
      return fail(MLA_ERR_INVALID_ARG, "unknown kv_dtype %d", p->kv_dtype);
  }
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
  if (pl.P > 1) {
    // few rows with many parts each: four waves per row
    if ((int64_t)pl.P >= 16 * (int64_t)p->batch)
      hipLaunchKernelGGL(mla_split_combine_kernel<4>, dim3(p->batch, pl.M), dim3(kThreads), 0, stream, dp);
    else
      hipLaunchKernelGGL(mla_split_combine_kernel<1>, dim3(p->batch, (pl.M + 3) / 4), dim3(kThreads), 0,
                         stream, dp);
    e = hipGetLastError();
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "combine launch: %s", hipGetErrorString(e));
  }
  return ok();
}

}  // namespace

extern "C" {

mla_status mla_combine(int32_t num_splits, int64_t rows, const float* partial_out,
                       const float* partial_lse, void* out, float* lse, hipStream_t stream) {
  if (num_splits < 1) return fail(MLA_ERR_INVALID_ARG, "num_splits must be >= 1");
  if (rows < 0) return fail(MLA_ERR_INVALID_ARG, "rows must be >= 0");
  if (rows == 0) return ok();
  if (!partial_out || !partial_lse || !out || !lse)
    return fail(MLA_ERR_INVALID_ARG, "null array argument");
  if (!aligned(partial_out, 16) || !aligned(out, 16) || !aligned(partial_lse, 4) ||
      !aligned(lse, 4))
    return fail(MLA_ERR_INVALID_ARG, "partial_out and out must be 16-byte aligned, lse arrays 4");
  if (rows > (int64_t)INT32_MAX * 4) return fail(MLA_ERR_UNSUPPORTED, "too many rows");
  hipLaunchKernelGGL(mla_combine_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(kThreads), 0,
                     stream, num_splits, rows, partial_out, partial_lse, (uint16_t*)out, lse);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "combine launch: %s", hipGetErrorString(e));
  return ok();
}

mla_status mla_plan(const mla_problem* p, const int32_t* seqlens, int32_t* plan_out,
                    int64_t plan_capacity, hipStream_t stream) {
  Plan pl;
  mla_status s = make_plan(p, &pl);
  if (s != MLA_OK) return s;
  const int64_t need = 3 * (int64_t)p->batch + pl.P + 2;
  if (!plan_out || (!seqlens && p->batch > 0))
    return fail(MLA_ERR_INVALID_ARG, "null array argument");
  if (plan_capacity < need)
    return fail(MLA_ERR_INVALID_ARG, "plan_out needs %lld int32 values",
                (long long)need);
  if (!aligned(plan_out, 4) || !aligned(seqlens, 4))
    return fail(MLA_ERR_INVALID_ARG, "plan_out and seqlens must be 4-byte aligned");
  hipLaunchKernelGGL(mla_plan_kernel, dim3(1), dim3(kThreads), 0, stream, seqlens, p->batch,
                     p->max_blocks_per_seq, pl.P, plan_out);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "plan launch: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
