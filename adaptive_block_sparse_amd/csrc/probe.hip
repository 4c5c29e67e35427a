// Sustained bf16 MFMA rate and shader clock of the chip, and the rate of the
// attention kernel's inner arithmetic on its own (measurement aids for the
// attention kernel's roofline; see abs_probe.h).
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

// The attention kernel's per-subtile arithmetic on its own: no K/V copies, no
// barrier, no padding, no work items.  Each round is one 32-key subtile:
//   softmax of the previous round's scores (exp2 of the float32 products,
//     four partial row sums, bf16 conversion to the PV operands),
//   scores S^T = K Q^T: 8 K operand reads from LDS, each feeding NG products
//     (NG groups of 32 queries held by the wave),
//   O^T += Vt P^T: 8 V operand reads from LDS, each feeding NG products.
// The LDS buffer holds small bf16 values, so scores stay within a few units
// and the exponentials finite.  NG = 1: 8 waves a workgroup (two per SIMD,
// the attention kernel's layout); NG = 2: 4 waves (one per SIMD, 64 queries).
constexpr int LOOP_LDS = 48 * 1024;

template <int NG>
__global__ __launch_bounds__(NG == 1 ? 512 : 256)
    __attribute__((amdgpu_waves_per_eu(3 - NG, 3 - NG))) void attn_loop_kernel(
        int iters, float* __restrict__ out, int64_t* __restrict__ clocks) {
  constexpr int NT = NG == 1 ? 512 : 256;
  __shared__ __attribute__((aligned(1024))) __bf16 lds[LOOP_LDS / 2];
  const int tid = threadIdx.x, lane = tid & 63;
  for (int i = tid; i < LOOP_LDS / 2; i += NT)
    lds[i] = (__bf16)((float)((i * 37) % 97) * (1.0f / 256.0f) - 0.1f);
  __syncthreads();
  // (the groups' operands differ at every k, so no product repeats another)
  bf16x8_t q[NG][8];
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        q[g][k][e] = (__bf16)((float)((lane + (2 * g + 1) * k + 5 * g + e) % 13) * 0.01f);
  f32x16_t o[NG][4], sp[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
#pragma unroll
    for (int e = 0; e < 16; ++e) sp[g][e] = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[g][u][e] = 0.f;
  }
  float l[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) l[g] = 0.f;
  // per-lane byte offsets of the A operands (two 16-byte halves of 32 rows)
  const int kread = (lane >> 5) * 2048 + (lane & 31) * 16;
  const int vread = 32768 + (lane >> 5) * 2048 + (lane & 31) * 16;
  const char* base = reinterpret_cast<const char*>(lds);
  const int64_t c0 = (int64_t)clock64(), w0 = (int64_t)wall_clock64();
  for (int it = 0; it < iters; ++it) {
    const int tb = (it & 3) * 512;   // K: 2.5 KB + 28 KB + 1.5 KB stays below 32 KB
    bf16x8_t p[NG][2];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      float a[4];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float x = __builtin_amdgcn_exp2f(sp[g][e]);
        a[e & 3] = e < 4 ? x : a[e & 3] + x;
        p[g][e / 8][e % 8] = (__bf16)x;
      }
      l[g] += (a[0] + a[1]) + (a[2] + a[3]);
    }
    f32x16_t s[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int e = 0; e < 16; ++e) s[g][e] = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const bf16x8_t av = *reinterpret_cast<const bf16x8_t*>(base + kread + k * 4096 + tb);
#pragma unroll
      for (int g = 0; g < NG; ++g)
        s[g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, q[g][k], s[g], 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        // V: 32 KB + 2.5 KB + 7 KB + 4.5 KB stays below 48 KB
        const bf16x8_t av =
            *reinterpret_cast<const bf16x8_t*>(base + vread + (kk * 4 + u) * 1024 + tb * 3);
#pragma unroll
        for (int g = 0; g < NG; ++g)
          o[g][u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, p[g][kk], o[g][u], 0, 0, 0);
      }
#pragma unroll
    for (int g = 0; g < NG; ++g) sp[g] = s[g];
  }
  const int64_t c1 = (int64_t)clock64(), w1 = (int64_t)wall_clock64();
  float acc = 0.f;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    acc += l[g];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc += o[g][u][e];
  }
  out[blockIdx.x * NT + tid] = acc;
  if (tid == 0) {
    clocks[2 * blockIdx.x] = c1 - c0;
    clocks[2 * blockIdx.x + 1] = w1 - w0;
  }
}

}  // namespace

extern "C" int abs_probe_attn_loop(int32_t queries_per_wave, int32_t iters, int32_t workgroups,
                                   float* out, int64_t* clocks, void* stream) {
  if (iters <= 0 || workgroups <= 0 || workgroups > ABS_PROBE_MAX_WORKGROUPS || !out || !clocks ||
      (queries_per_wave != 32 && queries_per_wave != 64))
    return 1;
  if (queries_per_wave == 32)
    hipLaunchKernelGGL(attn_loop_kernel<1>, dim3(workgroups), dim3(512), 0, (hipStream_t)stream,
                       iters, out, clocks);
  else
    hipLaunchKernelGGL(attn_loop_kernel<2>, dim3(workgroups), dim3(256), 0, (hipStream_t)stream,
                       iters, out, clocks);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

extern "C" int abs_probe_mfma_bf16(int32_t iters, int32_t workgroups, float* out,
                                   int64_t* clocks, void* stream) {
  if (iters <= 0 || workgroups <= 0 || workgroups > ABS_PROBE_MAX_WORKGROUPS || !out || !clocks)
    return 1;
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
