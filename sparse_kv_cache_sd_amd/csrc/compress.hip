// A second page scorer from compressed keys ("SparDA: Sparse Decoupled
// Attention ...", summary, Section 3.1: a parameter-free selector mean-pools
// the keys into overlapping compressed representations, sums the per-head
// relevance over the GQA group and max-pools it to the block score;
// Appendix C: kernel 32, stride 16, 64-token blocks).
//
// Setup (not part of the decode step, like the page bounds): window j of
// (sequence b, KV head g) is the fp32 mean of the valid keys 16 j .. 16 j +
// 31, for j < ceil(n_b / 16), stored in logical order.
//
// Scoring: the relevance of window j summed over the group's heads is
// scale * <sum_h q_h, c_j> (the sum of dot products is the dot product with
// the summed query, so one product per window); page u scores the max over
// the P / 16 windows that start inside it.  Windows past the sequence are
// masked to -inf before the max.
#include "kernels.h"
#include "device.h"

namespace sdkv {

namespace {

constexpr int kCThreads = 256;
constexpr int kCIters = 4;  // window rows per lane group and wave in the scorer

template <typename T, int D>
__global__ __launch_bounds__(kCThreads) void compress_keys_kernel(CompressArgs a) {
  constexpr int LPW = D / 8;             // lanes per window, 8 channels each
  constexpr int WPB = kCThreads / LPW;   // windows per block
  const Dims& d = a.d;
  const GroupBlock gb = group_block(d.B * d.Hkv);
  const int g = gb.bg % d.Hkv, b = gb.bg / d.Hkv;
  const int j = gb.j * WPB + (int)threadIdx.x / LPW;
  const int c0 = ((int)threadIdx.x % LPW) * 8;
  const int n = clamp_len(a.seq_lens[b], d.max_seq);
  const int J = (n + 15) / 16;
  if (j >= J || j >= a.max_windows) return;
  const T* kp = static_cast<const T*>(a.k_pages);
  float sum[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  int cnt = 0;
  const int t_end = min(16 * j + 32, n);
  for (int t = 16 * j; t < t_end; ++t) {
    const int lp = t / d.P;
    const int phys = a.block_table[(int64_t)b * d.max_pages + lp];
    if (phys < 0 || phys >= d.num_pages) continue;  // a page that is not attended
    float v[8];
    load8(kp + (((int64_t)phys * d.Hkv + g) * d.P + (t - lp * d.P)) * D + c0, v);
#pragma unroll
    for (int c = 0; c < 8; ++c) sum[c] += v[c];
    ++cnt;
  }
  const float inv = cnt > 0 ? 1.f / (float)cnt : 0.f;
  float* out = a.ckeys + (((int64_t)b * d.Hkv + g) * a.max_windows + j) * D + c0;
  *reinterpret_cast<float4*>(out) =
      make_float4(sum[0] * inv, sum[1] * inv, sum[2] * inv, sum[3] * inv);
  *reinterpret_cast<float4*>(out + 4) =
      make_float4(sum[4] * inv, sum[5] * inv, sum[6] * inv, sum[7] * inv);
}

// Max over aligned groups of W consecutive window slots (slot = lane / LPW).
template <int LPW, int W>
__device__ __forceinline__ float window_group_max(float x) {
#pragma unroll
  for (int o = LPW; o < LPW * W; o <<= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

template <typename T, int D, int G, int PW>
__global__ __launch_bounds__(kCThreads) void score_compressed_kernel(CompressArgs a) {
  constexpr int LPW = D / 8;                 // lanes per window
  constexpr int SPW = 64 / LPW;              // window slots per wave
  constexpr int NW = kCThreads / 64;
  constexpr int WB = NW * kCIters * SPW;     // windows per block
  static_assert(SPW % PW == 0, "a page's windows lie in one wave");
  const Dims& d = a.d;
  const GroupBlock gb = group_block(d.B * d.Hkv);
  const int g = gb.bg % d.Hkv, b = gb.bg / d.Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int slot = lane / LPW, c0 = (lane % LPW) * 8;
  // the summed query of the group, 8 channels per lane
  float qs[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float v[8];
    load8(static_cast<const T*>(a.q) + ((int64_t)b * d.Hq + g * G + h) * D + c0, v);
#pragma unroll
    for (int c = 0; c < 8; ++c) qs[c] += v[c];
  }
  const float* ck = a.ckeys + ((int64_t)b * d.Hkv + g) * a.max_windows * D + c0;
  const int j0 = gb.j * WB + wave * kCIters * SPW;
  // every load issued before the first use (window index clamped)
  float4 lo[kCIters], hi[kCIters];
#pragma unroll
  for (int it = 0; it < kCIters; ++it) {
    const int j = min(j0 + it * SPW + slot, a.max_windows - 1);
    lo[it] = *reinterpret_cast<const float4*>(ck + (int64_t)j * D);
    hi[it] = *reinterpret_cast<const float4*>(ck + (int64_t)j * D + 4);
  }
  const int n = clamp_len(a.seq_lens[b], d.max_seq);
  const int J = (n + 15) / 16;
  const int U = (n + d.P - 1) / d.P;
  float* out = a.unit_scores + ((int64_t)b * d.Hkv + g) * d.max_pages;
#pragma unroll
  for (int it = 0; it < kCIters; ++it) {
    const int j = j0 + it * SPW + slot;
    float acc = qs[0] * lo[it].x;
    acc = fmaf(qs[1], lo[it].y, acc);
    acc = fmaf(qs[2], lo[it].z, acc);
    acc = fmaf(qs[3], lo[it].w, acc);
    acc = fmaf(qs[4], hi[it].x, acc);
    acc = fmaf(qs[5], hi[it].y, acc);
    acc = fmaf(qs[6], hi[it].z, acc);
    acc = fmaf(qs[7], hi[it].w, acc);
    acc = group_sum<LPW>(acc);
    float r = j < J ? acc * d.scale : -INFINITY;
    r = window_group_max<LPW, PW>(r);
    const int u = j / PW;
    if (lane % (LPW * PW) == 0 && u < U) out[u] = r;
  }
}

}  // namespace

int compressed_windows(const Dims& d) { return (d.max_seq + 15) / 16; }

hipError_t launch_compress_keys(const CompressArgs& a, hipStream_t st) {
  const Dims& d = a.d;
  if (a.max_windows != compressed_windows(d)) return hipErrorInvalidValue;
  bool ok = false;
  auto run = [&](auto t, auto dd) {
    using T = decltype(t);
    constexpr int D = decltype(dd)::value;
    constexpr int WPB = kCThreads / (D / 8);
    const dim3 grid((a.max_windows + WPB - 1) / WPB * d.Hkv * d.B);
    compress_keys_kernel<T, D><<<grid, kCThreads, 0, st>>>(a);
    ok = true;
  };
  if (d.dtype == kBF16 && d.D == 128) run(bf16_t{}, std::integral_constant<int, 128>{});
  else if (d.dtype == kBF16 && d.D == 64) run(bf16_t{}, std::integral_constant<int, 64>{});
  else if (d.dtype == kF32 && d.D == 128) run(float{}, std::integral_constant<int, 128>{});
  else if (d.dtype == kF32 && d.D == 64) run(float{}, std::integral_constant<int, 64>{});
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_score_compressed(const CompressArgs& a, hipStream_t st) {
  const Dims& d = a.d;
  if (a.max_windows != compressed_windows(d) || (d.P != 16 && d.P != 64))
    return hipErrorInvalidValue;
  const bool ok = dispatch_tdg(d.dtype, d.D, d.G, [&](auto t, auto dd, auto gg) {
    using T = decltype(t);
    constexpr int D = decltype(dd)::value;
    constexpr int G = decltype(gg)::value;
    constexpr int WB = (kCThreads / 64) * kCIters * (64 / (D / 8));
    const dim3 grid((a.max_windows + WB - 1) / WB * d.Hkv * d.B);
    if (d.P == 16)
      score_compressed_kernel<T, D, G, 1><<<grid, kCThreads, 0, st>>>(a);
    else if (d.P == 64)
      score_compressed_kernel<T, D, G, 4><<<grid, kCThreads, 0, st>>>(a);
  });
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace sdkv
