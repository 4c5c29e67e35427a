// Sustained bf16 MFMA rate and shader clock of the chip (measurement aid for
// the attention kernel's roofline; see abs_probe.h).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "abs_probe.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// Varied operands in [-1, 1) from a multiplicative hash of the element index:
// all-zero operands would switch less and draw less power than real data.
__device__ __forceinline__ float hashed_unit(unsigned x) {
  x *= 2654435761u;
  x ^= x >> 15;
  x *= 2246822519u;
  return (float)(x >> 8) * (1.0f / 8388608.0f) - 1.0f;
}

__global__ __launch_bounds__(256) void mfma_peak_kernel(int iters, float* __restrict__ out,
                                                        int64_t* __restrict__ clocks) {
  const unsigned tid = blockIdx.x * blockDim.x + threadIdx.x;
  bf16x8_t a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)hashed_unit(16u * tid + e);
    b[e] = (__bf16)hashed_unit(16u * tid + 8 + e);
  }
  f32x16_t acc[4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[k][e] = 0.f;
  const int64_t c0 = (int64_t)clock64(), w0 = (int64_t)wall_clock64();
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[k], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[k][e];
  const int64_t c1 = (int64_t)clock64(), w1 = (int64_t)wall_clock64();
  out[tid] = s;
  if (threadIdx.x == 0) {
    clocks[2 * blockIdx.x] = c1 - c0;
    clocks[2 * blockIdx.x + 1] = w1 - w0;
  }
}

}  // namespace

extern "C" int abs_probe_mfma_bf16(int32_t iters, int32_t workgroups, float* out,
                                   int64_t* clocks, void* stream) {
  if (iters <= 0 || workgroups <= 0 || !out || !clocks) return 1;
  hipLaunchKernelGGL(mfma_peak_kernel, dim3(workgroups), dim3(256), 0, (hipStream_t)stream,
                     iters, out, clocks);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

extern "C" int abs_probe_wall_clock_khz(int32_t* khz) {
  if (!khz) return 1;
  int dev = 0, v = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 4;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return 4;
  *khz = v;
  return 0;
}
