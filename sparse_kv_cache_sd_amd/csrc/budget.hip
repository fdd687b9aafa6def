// Stage 1b with a dropped-mass budget (token unit): per (sequence b, KV head
// g), keep the shortest prefix of the top-k order (decreasing group score,
// equal scores to the lower id) whose dense softmax mass left outside is at
// most max_dropped for every head of the group, capped at keep_count(U).
// The dropped mass of the discarded entries governs the error and is
// controlled in advance ("Where Activation Sparsity and KV-Cache Sparsity
// Cross in LLM Decoding", cards view, pre-hoc sparsity abstract); in token
// unit every logit exists after scoring, so it can be computed exactly.
//
// One block per (b, g), up to kMaxSelectOne units:
//   1. per head h: m_h = max_t s[h, t] and 1 / Z_h, Z_h = sum_t e^(s - m_h)
//      (block reductions in a fixed order);
//   2. a radix search on the order keys of the group scores, like topk.h,
//      whose 256-bin histograms also accumulate every head's softmax mass
//      p_h(t) = e^(s - m_h) / Z_h as 2^40 fixed-point integers: integer sums
//      do not depend on the order of the LDS atomics, so the result does not
//      depend on timing.  The interval narrows to the first bin (from the
//      top) whose inclusion leaves at most the target outside for every head;
//   3. when the interval is one key value, its units (ties) are taken in id
//      order, one wave scanning 64 ids at a time, until the target holds;
//   4. the kept list is the exact top-k of topk.h with that count.
#include "topk.h"

namespace sdkv {

namespace {

constexpr int kBT = 1024;              // threads per block
constexpr int kBW = kBT / 64;
constexpr int kBK = kMaxSelectOne / kBT;  // keys per thread
constexpr int kBBins = 256;
constexpr int kBMaxG = 8;
constexpr float kFix = 1099511627776.0f;  // 2^40

typedef unsigned long long u64;

// The histogram passes add into kMC interleaved copies (copy = lane % kMC,
// padded apart so that the copies of a counter sit in different banks), then
// sum them: LDS atomics to one word serialise, and the scores crowd a few
// bins.
constexpr int kMC = 4;
constexpr int kMassStride = kBMaxG * kBBins + 1;  // u64 per copy
constexpr int kCntStride = kBBins + 1;            // words per copy

struct BudgetShared {
  RadixState rs;
  KeptScratch<kBK, kBW> ks;
  u64 mass[kBMaxG][kBBins];  // summed over the copies
  uint32_t cnt[kBBins];
  u64 massc[kMC * kMassStride];
  uint32_t cntc[kMC * kCntStride];
  float red[kBW];
  float m[kBMaxG], invz[kBMaxG];
  u64 tot[kBMaxG];    // all units' mass per head
  u64 above[kBMaxG];  // mass of the units above the interval
  uint32_t c_above;   // units above the interval
  uint32_t lo, hi;
  int kstar;          // > 0 once the count is known
};

__device__ __forceinline__ float block_max(BudgetShared& sm, float x) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  x = wave_max(x);
  if (lane == 0) sm.red[wave] = x;
  __syncthreads();
  float r = sm.red[0];
#pragma unroll
  for (int w = 1; w < kBW; ++w) r = fmaxf(r, sm.red[w]);
  __syncthreads();
  return r;
}

__device__ __forceinline__ float block_sum(BudgetShared& sm, float x) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  x = wave_sum(x);
  if (lane == 0) sm.red[wave] = x;
  __syncthreads();
  float r = 0.f;
#pragma unroll
  for (int w = 0; w < kBW; ++w) r += sm.red[w];
  __syncthreads();
  return r;
}

// VEC: rows of max_seq floats are 16-byte aligned (max_seq % 4 == 0).
template <bool VEC>
__global__ __launch_bounds__(kBT) void select_budget_kernel(BudgetArgs a) {
  __shared__ BudgetShared sm;
  const Dims& d = a.d;
  const int g = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = d.G;
  const int64_t bg = (int64_t)b * d.Hkv + g;
  const float* sc = a.scores + bg * a.U_max;
  const float* lg = a.logits + ((int64_t)b * d.Hq + (int64_t)g * G) * d.max_seq;
  const int n = clamp_len(a.seq_lens[b], d.max_seq);
  const int U = min(n, a.U_max);
  const int kcap = min(keep_count_dev(U, a.R_ppm), a.k_max);
  int32_t* out = a.sel_idx + bg * a.k_max;
  if (kcap == 0) {
    if (tid == 0) a.sel_count[bg] = 0;
    return;
  }
  // The normaliser and histogram passes take the tokens in groups of four
  // consecutive ones per thread (thread t, group j: tokens 4 (t + kBT j) ..
  // +3), read with 16-byte loads when the rows allow it; one CU has to pull
  // every logit of the group, so bytes in flight per load matter.  Group
  // starts are clamped to a valid group and masked afterwards, so every load
  // is issued unconditionally.
  constexpr int kGroups = kBK / 4;
  const int last_group = (U - 1) & ~3;
  auto ld4 = [&](const float* row, int t0) -> float4 {
    if constexpr (VEC) {
      return *reinterpret_cast<const float4*>(row + t0);
    } else {
      return make_float4(row[min(t0, U - 1)], row[min(t0 + 1, U - 1)], row[min(t0 + 2, U - 1)],
                         row[min(t0 + 3, U - 1)]);
    }
  };
  auto el = [](const float4& v, int i) { return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w; };
  // 1. dense softmax normalisers of the group's heads
  float acc[kBMaxG];
  for (int pass = 0; pass < 2; ++pass) {  // 0: max, 1: sum of exponentials
#pragma unroll
    for (int h = 0; h < kBMaxG; ++h) acc[h] = pass == 0 ? -INFINITY : 0.f;
    for (int j = 0; j < kGroups; j += 2) {  // two groups' loads in flight
#pragma unroll
      for (int h = 0; h < kBMaxG; ++h) {
        if (h >= G) break;
        float4 v[2];
#pragma unroll
        for (int q = 0; q < 2; ++q)
          v[q] = ld4(lg + (int64_t)h * d.max_seq, min(4 * (tid + kBT * (j + q)), last_group));
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int t0 = 4 * (tid + kBT * (j + q));
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (t0 + i >= U) continue;
            acc[h] = pass == 0 ? fmaxf(acc[h], el(v[q], i))
                               : acc[h] + exp2f((el(v[q], i) - sm.m[h]) * kLog2e);
          }
        }
      }
    }
    for (int h = 0; h < G; ++h) {
      const float r = pass == 0 ? block_max(sm, acc[h]) : block_sum(sm, acc[h]);
      if (tid == 0) {
        if (pass == 0) sm.m[h] = r;
        else sm.invz[h] = 1.f / r;
      }
    }
    __syncthreads();
  }
  // the target as a fixed-point mass
  const u64 target = (u64)(fminf(fmaxf(a.max_dropped, 0.f), 1.f) * kFix);
  auto weight_of = [&](int h, float s) -> u64 {
    const float w = exp2f((s - sm.m[h]) * kLog2e) * sm.invz[h];
    return (u64)(fminf(w, 1.f) * kFix);
  };
  auto weight = [&](int h, int t) -> u64 { return weight_of(h, lg[(int64_t)h * d.max_seq + t]); };
  // 2. radix search with mass histograms
  uint32_t mn = 0xFFFFFFFFu, mxk = 0u;
  for (int j = 0; j < kGroups; ++j) {
    const int t0 = 4 * (tid + kBT * j);
    const float4 v = ld4(sc, min(t0, last_group));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (t0 + i >= U) continue;
      const uint32_t k = order_key(el(v, i));
      mn = min(mn, k);
      mxk = max(mxk, k);
    }
  }
  block_minmax<kBW>(sm.rs, mn, mxk);
  if (tid == 0) {
    sm.lo = sm.rs.lo;
    sm.hi = sm.rs.hi;
    sm.c_above = 0u;
    sm.kstar = 0;
  }
  if (tid < kBMaxG) sm.above[tid] = 0ull;
  __syncthreads();
  bool first = true;
  while (sm.kstar == 0 && sm.lo != sm.hi) {
    const uint32_t lo = sm.lo, hi = sm.hi;
    const uint32_t shift = bin_shift(lo, hi);
    for (int i = tid; i < kMC * kMassStride; i += kBT) sm.massc[i] = 0ull;
    for (int i = tid; i < kMC * kCntStride; i += kBT) sm.cntc[i] = 0u;
    __syncthreads();
    u64* mrow = sm.massc + (lane % kMC) * kMassStride;
    uint32_t* crow = sm.cntc + (lane % kMC) * kCntStride;
    for (int j = 0; j < kGroups; ++j) {
      const int t0 = 4 * (tid + kBT * j), tc = min(t0, last_group);
      const float4 sv = ld4(sc, tc);
      uint32_t cm = 0u, bin[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t k = order_key(el(sv, i));
        bin[i] = (k - lo) >> shift;
        if (t0 + i < U && k >= lo && k <= hi) cm |= 1u << i;
      }
      if (cm == 0u) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if ((cm >> i) & 1u) atomicAdd(&crow[bin[i]], 1u);
#pragma unroll
      for (int h = 0; h < kBMaxG; ++h) {
        if (h >= G) break;
        const float4 v = ld4(lg + (int64_t)h * d.max_seq, tc);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if ((cm >> i) & 1u) atomicAdd(&mrow[h * kBBins + bin[i]], weight_of(h, el(v, i)));
      }
    }
    __syncthreads();
    for (int i = tid; i < kBBins; i += kBT) {
      uint32_t c = 0u;
#pragma unroll
      for (int q = 0; q < kMC; ++q) c += sm.cntc[q * kCntStride + i];
      sm.cnt[i] = c;
    }
    for (int i = tid; i < kBMaxG * kBBins; i += kBT) {
      u64 m = 0ull;
#pragma unroll
      for (int q = 0; q < kMC; ++q) m += sm.massc[q * kMassStride + i];
      sm.mass[i / kBBins][i % kBBins] = m;
    }
    __syncthreads();
    if (first) {  // every unit is in the first interval: the totals
      if (tid < G) {
        u64 s = 0ull;
        for (int i = 0; i < kBBins; ++i) s += sm.mass[tid][i];
        sm.tot[tid] = s;
      }
      __syncthreads();
      first = false;
      // keeping no unit already meets the target: one unit is kept (the
      // descent below needs a head above the target with the units above
      // the interval alone, or it would pick an empty top bin)
      bool met = true;
      for (int h = 0; h < G; ++h) met = met && sm.tot[h] <= target;
      if (met) {
        if (tid == 0) sm.kstar = 1;
        __syncthreads();
        break;
      }
    }
    if (wave == 0) {
      // lane l holds bins 255 - 4l - j (j < 4): descending order.  ok[j]:
      // keeping everything from bin 255 - 4l - j up meets the target for
      // every head
      bool ok[4] = {true, true, true, true};
      for (int h = 0; h < G; ++h) {
        u64 mb[4], s = 0ull;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          mb[j] = sm.mass[h][255 - 4 * lane - j];
          s += mb[j];
        }
        u64 run = sm.above[h] + (wave_incl_scan<u64>(s) - s);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          run += mb[j];
          if (sm.tot[h] > run + target) ok[j] = false;
        }
      }
      int hit = -1;
#pragma unroll
      for (int j = 3; j >= 0; --j)
        if (ok[j]) hit = j;
      const uint64_t hits = __ballot(hit >= 0);
      // the first bin meeting the target (the lowest bin as a guard: keeping
      // the whole interval always meets it)
      const int fl = hits ? (int)__builtin_ctzll(hits) : 63;
      const int fj = __shfl(hit >= 0 ? hit : 3, fl, 64);
      const uint32_t bin = (uint32_t)(255 - 4 * fl - fj);
      // units and mass in the bins above the chosen one
      uint32_t c_up = 0u;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (lane < fl || (lane == fl && j < fj)) c_up += sm.cnt[255 - 4 * lane - j];
      c_up = wave_sum(c_up);
      for (int h = 0; h < G; ++h) {
        u64 m_up = 0ull;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (lane < fl || (lane == fl && j < fj)) m_up += sm.mass[h][255 - 4 * lane - j];
        m_up = wave_incl_scan<u64>(m_up);
        if (lane == 63) sm.above[h] += m_up;
      }
      if (lane == 0) {
        const uint32_t nlo = lo + (bin << shift);
        const uint64_t top = (uint64_t)nlo + ((1ull << shift) - 1ull);
        sm.lo = nlo;
        sm.hi = (uint32_t)(top < (uint64_t)hi ? top : (uint64_t)hi);
        sm.c_above += c_up;
        // a bin of one unit: the count is known
        if (sm.cnt[bin] == 1u) sm.kstar = (int)(sm.c_above + 1u);
      }
    }
    __syncthreads();
  }
  if (first) {  // every key was equal: no histogram pass ran, sum the totals
    if (tid < kBMaxG) sm.tot[tid] = 0ull;
    __syncthreads();
    for (int h = 0; h < G; ++h) {
      u64 s = 0ull;
      for (int i = 0; i < kBK; ++i)
        if (tid + kBT * i < U) s += weight(h, tid + kBT * i);
      atomicAdd(&sm.tot[h], s);
    }
    __syncthreads();
  }
  // 3. ties: the units whose key is the interval's single value, in id order
  if (sm.kstar == 0) {
    const uint32_t T = sm.lo;
#pragma unroll
    for (int i = 0; i < kBK; ++i) {
      const int t = tid + kBT * i;
      const uint64_t tie = __ballot(t < U && order_key(sc[min(t, U - 1)]) == T);
      if (lane == 0) sm.ks.tie[i * kBW + wave] = tie;
    }
    __syncthreads();
    if (wave == 0) {
      u64 acc[kBMaxG];
#pragma unroll
      for (int h = 0; h < kBMaxG; ++h) acc[h] = sm.above[h];
      uint32_t taken = 0u;
      int found = 0;
      for (int e = 0; e < kBK * kBW && !found; ++e) {
        const uint64_t word = sm.ks.tie[e];
        if (word == 0ull) continue;
        const int u = 64 * e + lane;
        const bool mine = (word >> lane) & 1ull;
        bool ok = true;
        u64 tot_word[kBMaxG];
#pragma unroll
        for (int h = 0; h < kBMaxG; ++h) {
          const u64 w = (h < G && mine) ? weight(h, u) : 0ull;
          const u64 incl = wave_incl_scan<u64>(w);
          tot_word[h] = __shfl(incl, 63, 64);
          if (h < G && sm.tot[h] > acc[h] + incl + target) ok = false;
        }
        const uint64_t sat = __ballot(mine && ok);
        if (sat) {
          const int l = (int)__builtin_ctzll(sat);
          taken += (uint32_t)__popcll(word & ((2ull << l) - 1ull));
          found = 1;
        } else {
          taken += (uint32_t)__popcll(word);
#pragma unroll
          for (int h = 0; h < kBMaxG; ++h) acc[h] += tot_word[h];
        }
      }
      // every tie taken always meets the target (nothing is left outside
      // below T that the interval search had not already allowed)
      if (lane == 0) sm.kstar = (int)(sm.c_above + max(taken, 1u));
    }
    __syncthreads();
  }
  // 4. the exact top-k with that count
  const int k = max(1, min(sm.kstar, kcap));
  if (tid == 0) a.sel_count[bg] = k;
  if (k == U) {
    for (int i = tid; i < U; i += kBT) out[i] = i;
    return;
  }
  uint32_t key[kBK];
#pragma unroll
  for (int i = 0; i < kBK; ++i) key[i] = order_key(sc[min(tid + kBT * i, a.U_max - 1)]);
  topk_bitmap<kBK, kBW>(sm.rs, sm.ks, key, U, k);
  emit_kept<kBK, kBW>(sm.ks.mask, sm.ks.base, 0u, (uint32_t)k,
                      [&](int pos, int unit_id) { out[pos] = unit_id; });
}

}  // namespace

hipError_t launch_select_budget(const BudgetArgs& a, hipStream_t st) {
  if (a.U_max < 1 || a.U_max > kMaxSelectOne || a.d.G > kBMaxG || a.k_max < 1)
    return hipErrorInvalidValue;
  if ((a.d.max_seq & 3) == 0 && (a.U_max & 3) == 0)
    select_budget_kernel<true><<<dim3(a.d.Hkv, a.d.B), kBT, 0, st>>>(a);
  else
    select_budget_kernel<false><<<dim3(a.d.Hkv, a.d.B), kBT, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace sdkv
