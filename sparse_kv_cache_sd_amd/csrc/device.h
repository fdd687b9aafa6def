// Device helpers shared by the HIP kernels: storage conversion, 8-element row
// loads, wave-level shuffles and scans, and the template dispatcher.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "kernels.h"

namespace sdkv {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// bfloat16 is stored as its 16-bit pattern: the upper half of a binary32.
using bf16_t = uint16_t;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(bf16_t x) { return __uint_as_float(uint32_t(x) << 16); }

// Exact for values that are already representable in T (min / max of stored data).
template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t from_f<bf16_t>(float x) {
  return bf16_t(__float_as_uint(x) >> 16);
}

// Eight consecutive elements (16 bytes of bf16, 32 bytes of fp32) as floats.
__device__ __forceinline__ void load8(const bf16_t* p, float (&v)[8]) {
  const uint4 w = *reinterpret_cast<const uint4*>(p);
  v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x);
  v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
  v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z);
  v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
}
__device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

__device__ __forceinline__ int clamp_len(int n, int max_seq) {
  return n < 0 ? 0 : (n > max_seq ? max_seq : n);
}

// Inclusive prefix sum over the 64 lanes of a wavefront.
template <typename V>
__device__ __forceinline__ V wave_incl_scan(V v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const V t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}

// Calls fn(T{}, std::integral_constant<int, D>{}, std::integral_constant<int, G>{})
// for the supported (dtype, head_dim, group) combinations; returns false otherwise.
template <typename Fn>
bool dispatch_tdg(int dtype, int D, int G, Fn&& fn) {
  auto with_g = [&](auto t, auto d) -> bool {
    switch (G) {
      case 1: fn(t, d, std::integral_constant<int, 1>{}); return true;
      case 2: fn(t, d, std::integral_constant<int, 2>{}); return true;
      case 4: fn(t, d, std::integral_constant<int, 4>{}); return true;
      case 8: fn(t, d, std::integral_constant<int, 8>{}); return true;
      default: return false;
    }
  };
  auto with_d = [&](auto t) -> bool {
    switch (D) {
      case 64: return with_g(t, std::integral_constant<int, 64>{});
      case 128: return with_g(t, std::integral_constant<int, 128>{});
      default: return false;
    }
  };
  if (dtype == kF32) return with_d(float{});
  if (dtype == kBF16) return with_d(bf16_t{});
  return false;
}

}  // namespace sdkv
