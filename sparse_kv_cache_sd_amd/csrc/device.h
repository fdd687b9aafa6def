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

// Eight elements as raw 16-byte words, loaded now and widened later: keeping
// the load and the conversion apart lets a lane issue all of its loads before
// the first one is needed.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
template <typename T> struct Raw8 { u32x4_t w[sizeof(T) / 2]; };
template <typename T>
__device__ __forceinline__ Raw8<T> load_raw8(const T* p) {
  Raw8<T> r;
#pragma unroll
  for (int i = 0; i < (int)(sizeof(T) / 2); ++i) r.w[i] = reinterpret_cast<const u32x4_t*>(p)[i];
  return r;
}
__device__ __forceinline__ void widen8(const Raw8<bf16_t>& r, float (&v)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) { v[2 * i] = bf16_lo(r.w[0][i]); v[2 * i + 1] = bf16_hi(r.w[0][i]); }
}
__device__ __forceinline__ void widen8(const Raw8<float>& r, float (&v)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = __uint_as_float(r.w[i / 4][i % 4]);
}

// XCD-aware placement.  Workgroups are dealt to the eight XCDs round-robin by
// linear id, so a 1-D grid whose id is bg + BG * j (bg: the (sequence, KV
// head) index, j: the block's part of it) keeps every part of bg on XCD
// bg mod 8 when BG is a multiple of 8.  Data one kernel writes for bg and the
// next kernel reads (scores, partials, histograms) then stays in that XCD's
// L2 instead of being fetched across XCDs.  Only locality depends on this.
struct GroupBlock {
  int bg, j;
};
__device__ __forceinline__ GroupBlock group_block(int BG) {
  return GroupBlock{(int)(blockIdx.x % (unsigned)BG), (int)(blockIdx.x / (unsigned)BG)};
}

__device__ __forceinline__ int clamp_len(int n, int max_seq) {
  return n < 0 ? 0 : (n > max_seq ? max_seq : n);
}

// ---- cross-lane exchange without the LDS crossbar ----
// DPP moves within rows of 16 lanes: quad_perm xor 1 (0xB1), xor 2 (0x4E),
// row_half_mirror (lane i reads 7 - i within 8, 0x141), row_mirror (lane i
// reads 15 - i within 16, 0x140).  After the quad steps every lane of a quad
// holds the quad total, so a mirror pairs each lane with the other half.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of W lanes (W = 4, 8 or 16); every lane gets its group's total.
template <int W>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(W == 4 || W == 8 || W == 16, "group width");
  x += dpp_mov<0xB1>(x);
  x += dpp_mov<0x4E>(x);
  if constexpr (W >= 8) x += dpp_mov<0x141>(x);
  if constexpr (W >= 16) x += dpp_mov<0x140>(x);
  return x;
}

// Max over aligned groups of W lanes (W = 4, 8 or 16), same pairing as group_sum.
template <int W>
__device__ __forceinline__ float group_max(float x) {
  static_assert(W == 4 || W == 8 || W == 16, "group width");
  x = fmaxf(x, dpp_mov<0xB1>(x));
  x = fmaxf(x, dpp_mov<0x4E>(x));
  if constexpr (W >= 8) x = fmaxf(x, dpp_mov<0x141>(x));
  if constexpr (W >= 16) x = fmaxf(x, dpp_mov<0x140>(x));
  return x;
}

// gfx950 permlane swaps with old == src == x: the two results hold x of this
// lane and of lane ^ 32 (permlane32) or lane ^ 16 (permlane16), in an order
// that depends on the lane, so only symmetric combinations are formed.
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Inclusive prefix sum over the 64 lanes with DPP: row shifts by 1, 2, 4, 8
// (lanes without a source in their row add 0), then lane 15 of each row feeds
// the next row and lane 31 the upper half.
__device__ __forceinline__ uint32_t wave_scan_dpp(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, true);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, true);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, true);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, true);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);
  return v;
}

// Value of lane 63 broadcast to the wave.
__device__ __forceinline__ uint32_t wave_last(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Wave-wide unsigned min / max: DPP within rows of 16, permlane swaps across rows.
__device__ __forceinline__ uint32_t wave_umin(uint32_t v) {
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0xB1, 0xF, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x4E, 0xF, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x141, 0xF, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x140, 0xF, 0xF, false));
  auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  v = min(r[0], r[1]);
  r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return min(r[0], r[1]);
}
__device__ __forceinline__ uint32_t wave_umax(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0xB1, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x4E, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x141, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x140, 0xF, 0xF, false));
  auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  v = max(r[0], r[1]);
  r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return max(r[0], r[1]);
}

// Wave-wide max and sum (64 lanes) through the LDS crossbar; used off the hot loop.
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
__device__ __forceinline__ uint32_t wave_sum(uint32_t x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += (uint32_t)__shfl_xor((int)x, o);
  return x;
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

// alpha-entmax weight max(t, 0) ** beta of t = (alpha - 1) logit - tau, with
// beta = 1 / (alpha - 1): t^2 at alpha = 1.5, t at alpha = 2 (sparsemax).
// Every kernel forms t as fmaf(alpha - 1, logit, -tau), so the threshold
// kernel and the attention kernel weigh a token identically.
__device__ __forceinline__ float entmax_weight(float t, float beta) {
  if (!(t > 0.f)) return 0.f;
  if (beta == 2.f) return t * t;
  if (beta == 1.f) return t;
  return exp2f(beta * log2f(t));
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
