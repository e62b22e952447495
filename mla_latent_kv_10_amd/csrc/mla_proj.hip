// libmla, the steps either side of the decode kernel, for gfx950 (MI355X):
//  * query absorption   q~ = [W_UK[h]^T q_nope ; q_rope]     (128 -> 512 per head)
//  * output projection  o  = W_UV[h] o_lat                    (512 -> 128 per head)
//  * cache append       the new [c_KV | k_rope] rows of a decode step written
//                       into the paged cache (bf16, q8_0- or fp8-quantised)
// MLA recovers per-head keys and values from the cached latent through
// k = W_UK c and v = W_UV c ("MLA: Multi-Head Latent Attention -- DeepSeek-AI
// Explained", section Method); folding W_UK into the query and W_UV into the
// output (nnets.ru article, section on the essence of MLA; snowgate.dev forum
// thread 35, last reply) leaves these two small per-head products outside the
// attention kernel. The C ABI is in include/mla.h.
//
// Both products are per-head GEMMs with few rows (the decode batch) and a
// weight of 128 KiB per head, so they are bound by reading the weights once
// from HBM: each workgroup keeps its slice of one head's weight in registers
// as MFMA operands (32x32x16 bf16, fp32 accumulation) and streams that head's
// rows through it.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "mla.h"

namespace {

constexpr int kDL = MLA_D_LATENT;   // 512
constexpr int kDR = MLA_D_ROPE;     // 64
constexpr int kDK = MLA_D_K;        // 576
constexpr int kDH = MLA_D_HEAD;     // 128: per-head no-RoPE query / value width
constexpr int kBT = MLA_BLOCK_TOKENS;

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  typedef float f32x2v __attribute__((ext_vector_type(2)));
  const f32x2v f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2v));
}

__device__ __forceinline__ bf16x8 load16(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// 32x32 MFMA output layout: lane l holds column l % 32 and, in acc[4 g + r],
// row 8 g + 4 (l / 32) + r. Stores the 4 consecutive rows of group g of one
// column as bf16 (8 bytes).
__device__ __forceinline__ void store_group(uint16_t* dst, const f32x16& acc, int g) {
  const uint32_t w0 = pack_bf16x2(acc[4 * g + 0], acc[4 * g + 1]);
  const uint32_t w1 = pack_bf16x2(acc[4 * g + 2], acc[4 * g + 3]);
  *reinterpret_cast<uint64_t*>(dst) = (uint64_t)w0 | ((uint64_t)w1 << 32);
}

// Row tiles of a head are split over gridDim.z workgroups only as far as
// needed to give the chip about 512 workgroups: each split reads the head's
// weights again, and with 4 workgroups per head 128 heads already give 512.
unsigned row_splits(int64_t n_tok, int heads) {
  const int64_t tiles = (n_tok + 31) / 32;
  int64_t gz = (512 + 4 * (int64_t)heads - 1) / (4 * (int64_t)heads);
  if (gz > tiles) gz = tiles;
  if (gz > 8) gz = 8;
  return (unsigned)(gz < 1 ? 1 : gz);
}

// Query absorption. Workgroup (h, cb): latent columns 128 cb .. 128 cb + 127
// of head h, wave w the 32 columns d0 = 128 cb + 32 w. Per 32-row tile of the
// head's rows: D[d][t] = sum_j A[d][j] B[j][t], A = W_UK[h]^T (stored as
// w_uk_t[h][d][j], so a lane's 8 contraction values are contiguous), B = the
// rows' q_nope. The A fragments (8 k-steps, 32 VGPRs) stay in registers over
// all tiles. The tile's 32 x 128 outputs are staged in LDS so that each row's
// 256 bytes go out as whole 128-byte lines (stored from the MFMA layout, a
// lane's 8-byte pieces of 32 rows 147 KB apart would be written piecemeal).
// Workgroups with cb = 0 also copy the rows' q_rope (32 rows x 128 bytes per
// tile: one 16-byte piece per thread).
__global__ __launch_bounds__(256) void absorb_kernel(const uint16_t* __restrict__ q_nope,
                                                     const uint16_t* __restrict__ q_rope,
                                                     const uint16_t* __restrict__ w_uk_t,
                                                     uint16_t* __restrict__ q_abs,
                                                     int64_t n_tok, int H) {
  constexpr int kPad = 136;   // staged row: 128 outputs + 8 (16-byte aligned, spreads banks)
  __shared__ __attribute__((aligned(16))) uint16_t s_out[32 * kPad];
  const int h = blockIdx.x, cb = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l32 = lane & 31, hi = lane >> 5;
  const int d0 = 128 * cb + 32 * wave;
  bf16x8 af[8];
  const uint16_t* wrow = w_uk_t + ((int64_t)h * kDL + d0 + l32) * kDH + 8 * hi;
#pragma unroll
  for (int k = 0; k < 8; ++k) af[k] = load16(wrow + 16 * k);
  // the next tile's rows are loaded while this one is computed
  auto load_rows = [&](int64_t t0, bf16x8* bf) {
    const int64_t t = t0 + l32 < n_tok ? t0 + l32 : n_tok - 1;
    const uint16_t* qrow = q_nope + (t * H + h) * kDH + 8 * hi;
#pragma unroll
    for (int k = 0; k < 8; ++k) bf[k] = load16(qrow + 16 * k);
  };
  const int64_t tstep = (int64_t)gridDim.z * 32;
  bf16x8 bn[8];
  if ((int64_t)blockIdx.z * 32 < n_tok) load_rows((int64_t)blockIdx.z * 32, bn);
  for (int64_t t0 = (int64_t)blockIdx.z * 32; t0 < n_tok; t0 += tstep) {
    bf16x8 bf[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) bf[k] = bn[k];
    if (t0 + tstep < n_tok) load_rows(t0 + tstep, bn);
    // cb = 0 also copies the tile's q_rope (128 bytes per row, 8 lanes per
    // row, one 16-byte piece per thread): read now, written after the
    // outputs, so that the read's latency hides under the tile's work
    const int64_t tr = t0 + (threadIdx.x >> 3);
    const bool rope = cb == 0 && tr < n_tok;
    u32x4 rp = {};
    if (rope)
      rp = *reinterpret_cast<const u32x4*>(q_rope + (tr * H + h) * kDR + 8 * (threadIdx.x & 7));
    f32x16 acc = {};
#pragma unroll
    for (int k = 0; k < 8; ++k) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[k], bf[k], acc, 0, 0, 0);
#pragma unroll
    for (int g = 0; g < 4; ++g) store_group(s_out + l32 * kPad + 32 * wave + 8 * g + 4 * hi, acc, g);
    __syncthreads();
    // row r of the tile, 16-byte piece c (of 16): thread 16 r' + c, two rounds
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int u = threadIdx.x + 256 * i, r = u >> 4, c = u & 15;
      if (t0 + r < n_tok)
        *reinterpret_cast<u32x4*>(q_abs + ((t0 + r) * H + h) * kDK + 128 * cb + 8 * c) =
            *reinterpret_cast<const u32x4*>(s_out + r * kPad + 8 * c);
    }
    __syncthreads();
    if (rope) *reinterpret_cast<u32x4*>(q_abs + (tr * H + h) * kDK + kDL + 8 * (threadIdx.x & 7)) = rp;
  }
}

// Output projection. Workgroup (h, jb): output dims j = 32 jb .. 32 jb + 31 of
// head h; the 512-long contraction is split over the four waves (128 latent
// dims each), whose partial products are added in LDS in a fixed order.
// D[j][t] = sum_d A[j][d] B[d][t], A = W_UV[h] (row-major [128][512], a
// lane's 8 contraction values contiguous), B = the rows' o_lat.
__global__ __launch_bounds__(256) void project_kernel(const uint16_t* __restrict__ o_lat,
                                                      const uint16_t* __restrict__ w_uv,
                                                      uint16_t* __restrict__ o, int64_t n_tok,
                                                      int H) {
  __shared__ float red[3][16][64];
  const int h = blockIdx.x, jb = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l32 = lane & 31, hi = lane >> 5;
  const int kbase = 128 * wave;
  bf16x8 af[8];
  const uint16_t* wrow = w_uv + ((int64_t)h * kDH + 32 * jb + l32) * kDL + kbase + 8 * hi;
#pragma unroll
  for (int k = 0; k < 8; ++k) af[k] = load16(wrow + 16 * k);
  // the next tile's rows are loaded while this one is computed
  auto load_rows = [&](int64_t t0, bf16x8* bf) {
    const int64_t t = t0 + l32 < n_tok ? t0 + l32 : n_tok - 1;
    const uint16_t* orow_in = o_lat + (t * H + h) * kDL + kbase + 8 * hi;
#pragma unroll
    for (int k = 0; k < 8; ++k) bf[k] = load16(orow_in + 16 * k);
  };
  const int64_t tstep = (int64_t)gridDim.z * 32;
  bf16x8 bn[8];
  if ((int64_t)blockIdx.z * 32 < n_tok) load_rows((int64_t)blockIdx.z * 32, bn);
  for (int64_t t0 = (int64_t)blockIdx.z * 32; t0 < n_tok; t0 += tstep) {
    bf16x8 bf[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) bf[k] = bn[k];
    if (t0 + tstep < n_tok) load_rows(t0 + tstep, bn);
    f32x16 acc = {};
#pragma unroll
    for (int k = 0; k < 8; ++k) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[k], bf[k], acc, 0, 0, 0);
    if (wave > 0) {
#pragma unroll
      for (int i = 0; i < 16; ++i) red[wave - 1][i][lane] = acc[i];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = ((acc[i] + red[0][i][lane]) + red[1][i][lane]) + red[2][i][lane];
      if (t0 + l32 < n_tok) {
        uint16_t* dst = o + ((t0 + l32) * H + h) * kDH + 32 * jb + 4 * hi;
#pragma unroll
        for (int g = 0; g < 4; ++g) store_group(dst + 8 * g, acc, g);
      }
    }
    __syncthreads();
  }
}

// OCP E4M3 encoding of a finite float (1 sign, 4 exponent bits with bias 7,
// 3 fraction bits, no infinities, S.1111.111 = NaN): nearest, ties to even,
// saturated to +-448. Below 2^-6 the values are subnormal, steps of 2^-9.
__device__ __forceinline__ uint32_t e4m3_rne(float f) {
  const uint32_t sign = f < 0.0f || (f == 0.0f && signbit(f)) ? 0x80u : 0u;
  const float a = fabsf(f);
  if (a < 0.015625f) return sign | (uint32_t)rintf(a * 512.0f);
  int ex;
  frexpf(a, &ex);
  int e = ex - 1;
  float m = rintf(ldexpf(a, 3 - e));   // 8 .. 16
  if (m >= 16.0f) {
    m = 8.0f;
    ++e;
  }
  if (e > 8) return sign | 0x7Eu;
  const uint32_t code = (uint32_t)(((e + 7) << 3) | ((int)m - 8));
  return sign | (code == 0x7Fu ? 0x7Eu : code);
}

// Cache append: one wave per new row. Row i of sequence b is token
// t = seqlens[b] - s_q + i; positions outside the block table and block ids
// outside the pool are skipped (nothing is written for that row).
// bf16: the row is copied. q8_0: lane g < 18 quantises column group g
// (32 values): a = max |x|, d = a / 127 (fp32, correctly rounded), scale =
// fp16(d) to nearest even, code = x / d rounded half away from zero, clamped
// to [-127, 127]; a = 0 gives scale 0 and codes 0. q4_0 in Hadamard rotation:
// lane g < 18 takes block g (32 values), rotates it by H / sqrt(32) with the
// fast transform (strides 1, 2, 4, 8, 16: each pair (a, b) -> (a + b, a - b),
// then every value times the fp32 value of 1 / sqrt(32)), and writes its
// q4_0 encoding: m = the first value of largest magnitude, d = m / -8,
// code = min(15, floor(y / d + 8.5)) (all 8 when d = 0), scale fp16(d) to
// nearest even, codes two per byte (even code in the low nibble).
__global__ __launch_bounds__(64) void append_kernel(const uint16_t* __restrict__ rows,
                                                    const int32_t* __restrict__ block_table,
                                                    int max_blocks, const int32_t* __restrict__ seqlens,
                                                    int s_q, int64_t num_blocks, int kind,
                                                    uint8_t* __restrict__ kv,
                                                    uint16_t* __restrict__ scales) {
  const int64_t r = blockIdx.x;
  const int b = (int)(r / s_q), i = (int)(r % s_q);
  const int64_t t = (int64_t)seqlens[b] - s_q + i;
  if (t < 0 || t >= (int64_t)max_blocks * kBT) return;
  const int32_t blk = block_table[(int64_t)b * max_blocks + t / kBT];
  if (blk < 0 || (int64_t)blk >= num_blocks) return;
  const int64_t dst = (int64_t)blk * kBT + t % kBT;
  const uint16_t* src = rows + r * kDK;
  const int lane = threadIdx.x;
  if (kind == MLA_KV_BF16) {
    u32x4* d = reinterpret_cast<u32x4*>(kv + dst * kDK * 2);
    const u32x4* s = reinterpret_cast<const u32x4*>(src);
    for (int u = lane; u < kDK * 2 / 16; u += 64) d[u] = s[u];
    return;
  }
  if (kind == MLA_KV_FP8) {
    // one fp32 scale per token, d = max |x| / 448, code = E4M3(x / d): lane
    // l < 36 holds values 16 l .. 16 l + 15
    const bool act = lane < kDK / 16;
    float x[16];
    float amax = 0.0f;
    if (act) {
      const u32x4* s = reinterpret_cast<const u32x4*>(src + 16 * lane);
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const u32x4 w = s[c];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[8 * c + 2 * e] = __uint_as_float(w[e] << 16);
          x[8 * c + 2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
        }
      }
#pragma unroll
      for (int k = 0; k < 16; ++k) amax = fabsf(x[k]) > amax ? fabsf(x[k]) : amax;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
    const float d = amax / 448.0f;
    if (act) {
      uint32_t packed[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const uint32_t code = d > 0.0f ? e4m3_rne(x[k] / d) : 0u;
        packed[k >> 2] |= code << (8 * (k & 3));
      }
      *reinterpret_cast<u32x4*>(kv + dst * kDK + 16 * lane) =
          u32x4{packed[0], packed[1], packed[2], packed[3]};
      if (lane == 0) reinterpret_cast<float*>(scales)[dst] = d;
    }
    return;
  }
  if (kind == MLA_KV_Q4_0H) {
    if (lane >= kDK / MLA_Q8_GROUP) return;
    const u32x4* s = reinterpret_cast<const u32x4*>(src + MLA_Q8_GROUP * lane);
    float y[MLA_Q8_GROUP];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const u32x4 w = s[c];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        y[8 * c + 2 * e] = __uint_as_float(w[e] << 16);
        y[8 * c + 2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
      }
    }
#pragma unroll
    for (int st = 1; st < MLA_Q8_GROUP; st <<= 1)
#pragma unroll
      for (int k = 0; k < MLA_Q8_GROUP; ++k)
        if ((k & st) == 0) {
          const float a = y[k], b = y[k + st];
          y[k] = a + b;
          y[k + st] = a - b;
        }
    float m = 0.0f;
#pragma unroll
    for (int k = 0; k < MLA_Q8_GROUP; ++k) {
      y[k] = y[k] * 0.17677669529663688f;
      if (fabsf(y[k]) > fabsf(m)) m = y[k];
    }
    const float d = m / -8.0f;
    uint32_t packed[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < MLA_Q8_GROUP; ++k) {
      uint32_t c = 8u;
      if (d != 0.0f) {
        const float t = floorf(y[k] / d + 8.5f);
        c = t > 15.0f ? 15u : (uint32_t)(int)t;
      }
      packed[k >> 3] |= c << (4 * (k & 7));
    }
    *reinterpret_cast<u32x4*>(kv + dst * (kDK / 2) + 16 * lane) =
        u32x4{packed[0], packed[1], packed[2], packed[3]};
    scales[dst * (kDK / MLA_Q8_GROUP) + lane] = __builtin_bit_cast(uint16_t, (_Float16)d);
    return;
  }
  // q8_0
  if (lane >= kDK / MLA_Q8_GROUP) return;
  const u32x4* s = reinterpret_cast<const u32x4*>(src + MLA_Q8_GROUP * lane);
  float x[MLA_Q8_GROUP];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const u32x4 w = s[c];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[8 * c + 2 * e] = __uint_as_float(w[e] << 16);
      x[8 * c + 2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int k = 0; k < MLA_Q8_GROUP; ++k) amax = fabsf(x[k]) > amax ? fabsf(x[k]) : amax;
  const float d = amax / 127.0f;
  const _Float16 d16 = (_Float16)d;
  uint32_t packed[MLA_Q8_GROUP / 4];
#pragma unroll
  for (int k = 0; k < MLA_Q8_GROUP; ++k) {
    float c = 0.0f;
    if (d > 0.0f) c = roundf(x[k] / d);
    c = fminf(fmaxf(c, -127.0f), 127.0f);
    const uint32_t byte = (uint32_t)(uint8_t)(int8_t)(int)c;
    if ((k & 3) == 0) packed[k >> 2] = 0;
    packed[k >> 2] |= byte << (8 * (k & 3));
  }
  u32x4* qd = reinterpret_cast<u32x4*>(kv + dst * kDK + MLA_Q8_GROUP * lane);
  qd[0] = u32x4{packed[0], packed[1], packed[2], packed[3]};
  qd[1] = u32x4{packed[4], packed[5], packed[6], packed[7]};
  scales[dst * (kDK / MLA_Q8_GROUP) + lane] = __builtin_bit_cast(uint16_t, d16);
}

}  // namespace

// Errors of these entry points are reported through the error string of the
// decode entry points (mla_last_error), defined with them.
namespace mla_internal {
void set_last_error(const char* msg) __attribute__((visibility("hidden")));
}  // namespace mla_internal

namespace {
bool aligned_to(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }
void mla_set_last_error(const char* msg) { mla_internal::set_last_error(msg); }
}  // namespace

extern "C" {

mla_status mla_absorb_query(int64_t rows, int32_t num_heads, const void* q_nope,
                            const void* q_rope, const void* w_uk_t, void* q_abs,
                            hipStream_t stream) {
  if (rows < 0 || num_heads < 1 || rows % num_heads) {
    mla_set_last_error("rows must be a non-negative multiple of num_heads >= 1");
    return MLA_ERR_INVALID_ARG;
  }
  if (rows == 0) return MLA_OK;
  if (!q_nope || !q_rope || !w_uk_t || !q_abs) {
    mla_set_last_error("null array argument");
    return MLA_ERR_INVALID_ARG;
  }
  if (!aligned_to(q_nope, 16) || !aligned_to(q_rope, 16) || !aligned_to(w_uk_t, 16) ||
      !aligned_to(q_abs, 16)) {
    mla_set_last_error("arrays must be 16-byte aligned");
    return MLA_ERR_INVALID_ARG;
  }
  const int64_t n_tok = rows / num_heads;
  const unsigned gz = row_splits(n_tok, num_heads);
  hipLaunchKernelGGL(absorb_kernel, dim3(num_heads, 4, gz), dim3(256), 0, stream,
                     (const uint16_t*)q_nope, (const uint16_t*)q_rope, (const uint16_t*)w_uk_t,
                     (uint16_t*)q_abs, n_tok, num_heads);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    mla_set_last_error(hipGetErrorString(e));
    return MLA_ERR_HIP;
  }
  return MLA_OK;
}

mla_status mla_project_output(int64_t rows, int32_t num_heads, const void* o_lat,
                              const void* w_uv, void* o, hipStream_t stream) {
  if (rows < 0 || num_heads < 1 || rows % num_heads) {
    mla_set_last_error("rows must be a non-negative multiple of num_heads >= 1");
    return MLA_ERR_INVALID_ARG;
  }
  if (rows == 0) return MLA_OK;
  if (!o_lat || !w_uv || !o) {
    mla_set_last_error("null array argument");
    return MLA_ERR_INVALID_ARG;
  }
  if (!aligned_to(o_lat, 16) || !aligned_to(w_uv, 16) || !aligned_to(o, 16)) {
    mla_set_last_error("arrays must be 16-byte aligned");
    return MLA_ERR_INVALID_ARG;
  }
  const int64_t n_tok = rows / num_heads;
  const unsigned gz = row_splits(n_tok, num_heads);
  hipLaunchKernelGGL(project_kernel, dim3(num_heads, 4, gz), dim3(256), 0, stream,
                     (const uint16_t*)o_lat, (const uint16_t*)w_uv, (uint16_t*)o, n_tok,
                     num_heads);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    mla_set_last_error(hipGetErrorString(e));
    return MLA_ERR_HIP;
  }
  return MLA_OK;
}

mla_status mla_cache_append(int32_t batch, int32_t seqlen_q, const void* rows,
                            const int32_t* block_table, int32_t max_blocks_per_seq,
                            const int32_t* seqlens, int64_t num_blocks, int32_t kv_dtype,
                            void* kv_cache, void* kv_scales, hipStream_t stream) {
  if (batch < 0 || seqlen_q < 1 || max_blocks_per_seq < 1 || num_blocks < 0) {
    mla_set_last_error("batch >= 0, seqlen_q >= 1, max_blocks_per_seq >= 1, num_blocks >= 0");
    return MLA_ERR_INVALID_ARG;
  }
  if (kv_dtype != MLA_KV_BF16 && kv_dtype != MLA_KV_Q8_0 && kv_dtype != MLA_KV_FP8 &&
      kv_dtype != MLA_KV_Q4_0H) {
    mla_set_last_error("unknown kv_dtype");
    return MLA_ERR_INVALID_ARG;
  }
  if ((int64_t)max_blocks_per_seq * MLA_BLOCK_TOKENS > INT32_MAX) {
    mla_set_last_error("block table too large");
    return MLA_ERR_UNSUPPORTED;
  }
  if (batch == 0) return MLA_OK;
  if (!rows || !block_table || !seqlens || !kv_cache || (kv_dtype != MLA_KV_BF16 && !kv_scales)) {
    mla_set_last_error("null array argument");
    return MLA_ERR_INVALID_ARG;
  }
  if (!aligned_to(rows, 16) || !aligned_to(kv_cache, 16) || !aligned_to(block_table, 4) ||
      !aligned_to(seqlens, 4) || (kv_scales && !aligned_to(kv_scales, 4))) {
    mla_set_last_error("rows and kv_cache must be 16-byte aligned, the others 4");
    return MLA_ERR_INVALID_ARG;
  }
  hipLaunchKernelGGL(append_kernel, dim3((unsigned)((int64_t)batch * seqlen_q)),
                     dim3(64), 0, stream, (const uint16_t*)rows, block_table, max_blocks_per_seq,
                     seqlens, seqlen_q, num_blocks, kv_dtype, (uint8_t*)kv_cache,
                     (uint16_t*)kv_scales);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    mla_set_last_error(hipGetErrorString(e));
    return MLA_ERR_HIP;
  }
  return MLA_OK;
}

}  // extern "C"
