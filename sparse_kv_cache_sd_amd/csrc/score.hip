// Stage 1a: query-aware scoring of KV units.
//
// Page unit: an upper bound on each page's largest logit from the page's
// channel-wise key minima and maxima ("Where Activation Sparsity and KV-Cache
// Sparsity Cross in LLM Decoding", cards view, EntmaxKV abstract: pages are
// ranked from light statistics before they are loaded).  For one head,
// sum_c max(q_c kmin_c, q_c kmax_c) = sum_c q_c * (q_c >= 0 ? kmax_c : kmin_c)
// because kmin_c <= kmax_c, and rounding is monotone, so the selected product
// is also the larger one in floating point.  The group's score is the max over
// its G query heads.
//
// Token unit: the exact logits scale * q.K of every valid key, kept for the
// attention pass, and their max over the group ("... list view", Abstract:
// attention-scored KV selection reads every key once).
//
// Layout of work: one row (a page's bound pair, or a token's key) is read by
// LPR = d/8 consecutive lanes, 8 channels (16 B of bf16) each, so a wave
// reads 64/LPR rows per load; each lane holds its 8 channels of the group's
// G queries in registers, and partial sums are reduced across the LPR lanes.
#include "device.h"

namespace sdkv {

constexpr int kScoreThreads = 256;
constexpr int kScoreRowsPerBlock = 256;

template <typename T, int D, int G>
__global__ __launch_bounds__(kScoreThreads) void score_pages_kernel(
    const T* __restrict__ q, const T* __restrict__ bounds,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens,
    float* __restrict__ scores, Dims d) {
  constexpr int LPR = D / 8;
  constexpr int RPW = 64 / LPR;
  constexpr int NW = kScoreThreads / 64;
  const int g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane / LPR, cl = lane % LPR;
  const int n = clamp_len(seq_lens[b], d.max_seq);
  const int U = (n + d.P - 1) / d.P;
  const int u0 = blockIdx.x * kScoreRowsPerBlock;
  if (u0 >= U) return;
  const int u1 = min(U, u0 + kScoreRowsPerBlock);

  float qv[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
    load8(q + ((int64_t)b * d.Hq + g * G + h) * D + cl * 8, qv[h]);

  float* out = scores + ((int64_t)b * d.Hkv + g) * d.max_pages;
  for (int base = u0 + wave * RPW; base < u1; base += NW * RPW) {
    const int u = base + sub;
    bool ok = u < u1;
    int phys = ok ? block_table[(int64_t)b * d.max_pages + u] : -1;
    ok = ok && phys >= 0 && phys < d.num_pages;
    float lo[8], hi[8];
    if (ok) {
      const T* row = bounds + ((int64_t)phys * d.Hkv + g) * 2 * D + cl * 8;
      load8(row, lo);
      load8(row + D, hi);
    } else {
#pragma unroll
      for (int c = 0; c < 8; ++c) lo[c] = hi[c] = 0.f;
    }
    float best = -INFINITY;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) acc = fmaf(qv[h][c], qv[h][c] >= 0.f ? hi[c] : lo[c], acc);
#pragma unroll
      for (int o = LPR / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o, LPR);
      best = fmaxf(best, acc * d.scale);
    }
    // A page whose block-table entry is out of range ranks last.
    if (u < u1 && cl == 0) out[u] = ok ? best : -3.0e38f;
  }
}

template <typename T, int D, int G>
__global__ __launch_bounds__(kScoreThreads) void score_tokens_kernel(
    const T* __restrict__ q, const T* __restrict__ k_pages,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens,
    float* __restrict__ scores, float* __restrict__ logits, Dims d) {
  constexpr int LPR = D / 8;
  constexpr int RPW = 64 / LPR;
  constexpr int NW = kScoreThreads / 64;
  const int g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane / LPR, cl = lane % LPR;
  const int n = clamp_len(seq_lens[b], d.max_seq);
  const int t0 = blockIdx.x * kScoreRowsPerBlock;
  if (t0 >= n) return;
  const int t1 = min(n, t0 + kScoreRowsPerBlock);

  float qv[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
    load8(q + ((int64_t)b * d.Hq + g * G + h) * D + cl * 8, qv[h]);

  float* sc = scores + ((int64_t)b * d.Hkv + g) * d.max_seq;
  for (int base = t0 + wave * RPW; base < t1; base += NW * RPW) {
    const int t = base + sub;
    bool ok = t < t1;
    const int lp = t / d.P;
    int phys = ok ? block_table[(int64_t)b * d.max_pages + lp] : -1;
    ok = ok && phys >= 0 && phys < d.num_pages;
    float kv[8];
    if (ok) {
      load8(k_pages + (((int64_t)phys * d.Hkv + g) * d.P + (t - lp * d.P)) * D + cl * 8, kv);
    } else {
#pragma unroll
      for (int c = 0; c < 8; ++c) kv[c] = 0.f;
    }
    float best = -INFINITY, mine = 0.f;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) acc = fmaf(qv[h][c], kv[c], acc);
#pragma unroll
      for (int o = LPR / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o, LPR);
      const float s = acc * d.scale;
      best = fmaxf(best, s);
      if (h == cl) mine = s;
    }
    if (t < t1) {
      if (!ok) { best = -3.0e38f; mine = -3.0e38f; }
      if (cl < G) logits[((int64_t)b * d.Hq + g * G + cl) * d.max_seq + t] = mine;
      if (cl == 0) sc[t] = best;
    }
  }
}

hipError_t launch_score(const ScoreArgs& a, hipStream_t st) {
  const Dims& d = a.d;
  const int U_max = a.unit == kPage ? d.max_pages : d.max_seq;
  const dim3 grid((U_max + kScoreRowsPerBlock - 1) / kScoreRowsPerBlock, d.Hkv, d.B);
  const bool ok = dispatch_tdg(d.dtype, d.D, d.G, [&](auto t, auto dd, auto gg) {
    using T = decltype(t);
    constexpr int D = decltype(dd)::value;
    constexpr int G = decltype(gg)::value;
    if (a.unit == kPage) {
      score_pages_kernel<T, D, G><<<grid, kScoreThreads, 0, st>>>(
          static_cast<const T*>(a.q), static_cast<const T*>(a.bounds), a.block_table,
          a.seq_lens, a.unit_scores, d);
    } else {
      score_tokens_kernel<T, D, G><<<grid, kScoreThreads, 0, st>>>(
          static_cast<const T*>(a.q), static_cast<const T*>(a.k_pages), a.block_table,
          a.seq_lens, a.unit_scores, a.token_logits, d);
    }
  });
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace sdkv
