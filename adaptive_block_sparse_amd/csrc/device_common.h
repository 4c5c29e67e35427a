// Device helpers shared by the routing and attention kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace abs_impl {

typedef uint16_t bf16_t;  // raw bfloat16 bits

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Loads 16 bytes and widens them to float: 8 bf16 or 4 float values.
template <typename T> struct Chunk;
template <> struct Chunk<float> {
  static constexpr int E = 4;
  __device__ __forceinline__ static void load(const float* p, float* out) {
    float4 v = *reinterpret_cast<const float4*>(p);
    out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
  }
  __device__ __forceinline__ static void unpack(uint4 v, float* out) {
    out[0] = __uint_as_float(v.x); out[1] = __uint_as_float(v.y);
    out[2] = __uint_as_float(v.z); out[3] = __uint_as_float(v.w);
  }
};
template <> struct Chunk<bf16_t> {
  static constexpr int E = 8;
  __device__ __forceinline__ static void load(const bf16_t* p, float* out) {
    uint4 v = *reinterpret_cast<const uint4*>(p);
    out[0] = bf16_lo(v.x); out[1] = bf16_hi(v.x);
    out[2] = bf16_lo(v.y); out[3] = bf16_hi(v.y);
    out[4] = bf16_lo(v.z); out[5] = bf16_hi(v.z);
    out[6] = bf16_lo(v.w); out[7] = bf16_hi(v.w);
  }
  __device__ __forceinline__ static void unpack(uint4 v, float* out) {
    out[0] = bf16_lo(v.x); out[1] = bf16_hi(v.x);
    out[2] = bf16_lo(v.y); out[3] = bf16_hi(v.y);
    out[4] = bf16_lo(v.z); out[5] = bf16_hi(v.z);
    out[6] = bf16_lo(v.w); out[7] = bf16_hi(v.w);
  }
};

// Wave (64 lanes) reductions and scans through cross-lane shuffles.
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ __forceinline__ int wave_sum_int(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
template <typename V>
__device__ __forceinline__ V wave_inclusive_scan(V x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    V y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

// Block-wide exclusive scan of one value per thread (NT threads, NT/64 waves).
// `tmp` is shared scratch of at least NT/64 + 1 elements.  Returns the
// exclusive prefix; *total receives the block sum.
template <int NT, typename V>
__device__ __forceinline__ V block_exclusive_scan(V x, V* tmp, V* total) {
  constexpr int NWV = NT / 64;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  V inc = wave_inclusive_scan(x);
  if (lane == 63) tmp[wv] = inc;
  __syncthreads();
  if (threadIdx.x == 0) {
    V run = 0;
    for (int i = 0; i < NWV; ++i) { V t = tmp[i]; tmp[i] = run; run += t; }
    tmp[NWV] = run;
  }
  __syncthreads();
  V res = tmp[wv] + inc - x;
  *total = tmp[NWV];
  __syncthreads();
  return res;
}

template <int NT>
__device__ __forceinline__ float block_max(float x, float* tmp) {
  constexpr int NWV = NT / 64;
  x = wave_max(x);
  if ((threadIdx.x & 63) == 0) tmp[threadIdx.x >> 6] = x;
  __syncthreads();
  float r = tmp[0];
#pragma unroll
  for (int i = 1; i < NWV; ++i) r = fmaxf(r, tmp[i]);
  __syncthreads();
  return r;
}

template <int NT>
__device__ __forceinline__ float block_sum(float x, float* tmp) {
  constexpr int NWV = NT / 64;
  x = wave_sum(x);
  if ((threadIdx.x & 63) == 0) tmp[threadIdx.x >> 6] = x;
  __syncthreads();
  float r = tmp[0];
#pragma unroll
  for (int i = 1; i < NWV; ++i) r += tmp[i];
  __syncthreads();
  return r;
}

// Hardware identity of the executing wave's compute unit.
__device__ __forceinline__ uint32_t hw_id_reg() {
  return __builtin_amdgcn_s_getreg((31 << 11) | (0 << 6) | 4);   // HW_REG_HW_ID
}
__device__ __forceinline__ uint32_t xcc_id_reg() {
  return __builtin_amdgcn_s_getreg((31 << 11) | (0 << 6) | 20);  // HW_REG_XCC_ID
}

}  // namespace abs_impl
