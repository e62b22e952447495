// Measurement probes for libmla's profiles. The MFMA probe keeps every SIMD's
// matrix core busy with independent bf16 MFMAs (v_mfma_f32_32x32x16_bf16,
// 32768 flops each), so that its rate is the chip's sustained dense bf16
// MFMA rate and its counter readings (SQ_VALU_MFMA_BUSY_CYCLES against
// GRBM_GUI_ACTIVE) calibrate what "fully busy" reads as. The LDS probe
// measures the rate at which waves receive LDS data. Not part of the decode
// path; built into their own library (libmlaprobe.so).
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));

// One wave per SIMD (256 threads per workgroup); each wave runs `iters`
// rounds of 8 independent MFMAs (8 accumulators, so no MFMA waits on the
// previous one) and stores a checksum so nothing is optimised away.
__global__ __launch_bounds__(256, 1) void mfma_probe_kernel(float* out, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (lane + i));
    b[i] = (__bf16)(0.002f * (lane - i));
  }
  f32x16 acc[8];
  for (int j = 0; j < 8; ++j)
    for (int i = 0; i < 16; ++i) acc[j][i] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.f;
  for (int j = 0; j < 8; ++j)
    for (int i = 0; i < 16; ++i) s += acc[j][i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// LDS read rate: WAVES waves per workgroup (one workgroup per CU, 64 KiB of
// LDS), each wave issuing 8 independent ds_read_b128 per round from its own
// 4 KiB window (consecutive lanes, consecutive 16 bytes: no bank conflicts),
// timed per wave in shader cycles (s_memtime). out[4 (wg * WAVES + w)] gets
// the wave's cycles, the next word a checksum.
typedef uint32_t u32x4p __attribute__((ext_vector_type(4)));
template <int WAVES>
__global__ __launch_bounds__(64 * WAVES, 1) void lds_probe_kernel(uint32_t* out, int iters) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[65536];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  for (int i = t; i < 65536 / 16; i += 64 * WAVES)
    reinterpret_cast<u32x4p*>(lds)[i] = u32x4p{(uint32_t)i, 1u, 2u, 3u};
  __syncthreads();
  u32x4p acc[8];
  for (int j = 0; j < 8; ++j) acc[j] = u32x4p{0u, 0u, 0u, 0u};
  const uint32_t base = (uint32_t)(4096 * w + 16 * lane);
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j)   // masked to the 64 KiB array, 16-byte aligned
      acc[j] ^= *reinterpret_cast<const u32x4p*>(lds + ((base + 1024u * j + 16384u * (it & 3)) & 65535u));
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  u32x4p x = acc[0];
  for (int j = 1; j < 8; ++j) x ^= acc[j];
  if (lane == 0) {
    out[4 * (blockIdx.x * WAVES + w)] = (uint32_t)(t1 - t0);
    out[4 * (blockIdx.x * WAVES + w) + 1] = x[0] ^ x[1] ^ x[2] ^ x[3];
  }
}

extern "C" {

// LDS read-rate probe on `stream`: `workgroups` x (64 * waves) threads, waves
// in {1, 2, 4, 8}, `iters` rounds of 8 ds_read_b128 per wave (1 KiB each). out: device buffer of workgroups * waves * 4
// words. Returns a hipError_t value (hipErrorInvalidValue for other waves).
int mla_probe_lds(uint32_t* out, int workgroups, int waves, int iters, hipStream_t stream) {
  switch (waves) {
    case 1: hipLaunchKernelGGL(lds_probe_kernel<1>, dim3(workgroups), dim3(64), 0, stream, out, iters); break;
    case 2: hipLaunchKernelGGL(lds_probe_kernel<2>, dim3(workgroups), dim3(128), 0, stream, out, iters); break;
    case 4: hipLaunchKernelGGL(lds_probe_kernel<4>, dim3(workgroups), dim3(256), 0, stream, out, iters); break;
    case 8: hipLaunchKernelGGL(lds_probe_kernel<8>, dim3(workgroups), dim3(512), 0, stream, out, iters); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

// Launch the probe on `stream`: `workgroups` x 256 threads, `iters` rounds of
// 8 MFMAs per wave (flops = workgroups * 4 * iters * 8 * 32768). out: device
// buffer of workgroups * 256 floats. Returns a hipError_t value.
int mla_probe_mfma(float* out, int workgroups, int iters, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(workgroups), dim3(256), 0, stream, out, iters);
  return (int)hipGetLastError();
}

}  // extern "C"
