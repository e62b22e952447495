// Measurement probe for libmla's profiles: a kernel that keeps every SIMD's
// matrix core busy with independent bf16 MFMAs (v_mfma_f32_32x32x16_bf16,
// 32768 flops each), so that its rate is the chip's sustained dense bf16
// MFMA rate and its counter readings (SQ_VALU_MFMA_BUSY_CYCLES against
// GRBM_GUI_ACTIVE) calibrate what "fully busy" reads as. Not part of the
// decode path; built into its own library (libmlaprobe.so).
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

extern "C" {

// Launch the probe on `stream`: `workgroups` x 256 threads, `iters` rounds of
// 8 MFMAs per wave (flops = workgroups * 4 * iters * 8 * 32768). out: device
// buffer of workgroups * 256 floats. Returns a hipError_t value.
int mla_probe_mfma(float* out, int workgroups, int iters, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(workgroups), dim3(256), 0, stream, out, iters);
  return (int)hipGetLastError();
}

}  // extern "C"
