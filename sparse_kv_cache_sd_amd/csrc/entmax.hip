// alpha-entmax threshold over the kept tokens of every (sequence, query head).
//
// "Where Activation Sparsity and KV-Cache Sparsity Cross in LLM Decoding",
// cards view, EntmaxKV abstract: alpha-entmax attention has exact zeros, so
// sparse decoding over kept candidates that hold its support is exact.  The
// weights over a kept set T are p_t = max((alpha - 1) z_t - tau, 0) ** beta,
// beta = 1 / (alpha - 1), with tau chosen so that they sum to one over T.
//
// Root finding.  With t_i = (alpha - 1) z_i - tau and S0 = sum max(t_i, 0)^beta,
// the root of S0 = 1 is the root of g(tau) = S0^(1/beta) - 1, the beta-norm of
// the positive parts minus one.  g is convex and decreasing in tau (a norm,
// monotone in each entry, of entries that are convex and decreasing in tau),
// g((alpha - 1) max z - 1) >= 0, and g is linear when the positive t_i are
// equal.  Newton steps on g from that left end therefore climb monotonically
// to the root (the tangent of a convex decreasing function lies below it):
//   tau += (S0 - S0^(2 - alpha)) / S1,   S1 = sum max(t_i, 0)^(beta - 1),
// a handful of steps for any alpha in (1, 2] (sparsemax ends exactly).  The
// iteration stops once S0 <= 1 (the root, up to rounding) or a step no longer
// moves tau.  Every later tau is >= the first, so tokens with t_i <= 0 there
// weigh 0 from then on and only the others ("candidates") take part.
//
// One 1024-thread block per (sequence, query head); block id
// bg + B * H_kv * (h mod G) puts the G heads of a KV head on the XCD that
// runs the attention blocks of that KV head.  The block gathers the kept
// logits (the first 16384 into registers, 16 per thread), finds their max,
// and compacts the candidates into LDS in slot order (wave ballots and
// prefix offsets, so the order -- and with it every fp32 sum -- does not
// depend on timing).  One wave then runs the Newton steps over the compacted
// candidates with wave-level sums only.  With more than kTauCap candidates
// the whole block iterates instead, over its registers and the rest of the
// logits, re-read each step.
#include "device.h"

namespace sdkv {

constexpr int kTauThreads = 1024;
constexpr int kTauKeys = 16;     // logits per thread held in registers
constexpr int kTauCap = 12288;   // candidates compacted into LDS (48 KB)
constexpr int kTauBatch = 8;     // tail rounds whose loads are issued together

// Sum and max over the 64 lanes without the LDS crossbar: DPP within rows of
// 16, then the gfx950 permlane swaps across rows.  Every lane gets the result.
__device__ __forceinline__ float wave_sum_dpp(float x) {
  x = group_sum<16>(x);
  x = sum_xor16(x);
  return sum_xor32(x);
}
__device__ __forceinline__ float wave_max_dpp(float x) {
  x = group_max<16>(x);
  x = max_xor16(x);
  return max_xor32(x);
}

__global__ __launch_bounds__(kTauThreads) void entmax_tau_kernel(TauArgs a) {
  constexpr int NT = kTauThreads, NW = NT / 64, KPT = kTauKeys;
  __shared__ float s_c[kTauCap];
  __shared__ float s_red[2][2][NW];
  __shared__ float s_max[NW];
  __shared__ int s_cnt[NW];
  const Dims& d = a.d;
  const GroupBlock gb = group_block(d.B * d.Hkv);
  const int g = gb.bg % d.Hkv, b = gb.bg / d.Hkv, h = g * d.G + gb.j;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = clamp_len(a.seq_lens[b], d.max_seq);
  const bool pg = a.unit == kPage;
  const int U = pg ? (n + d.P - 1) / d.P : n;
  const int32_t* list = a.sel_idx ? a.sel_idx + (int64_t)gb.bg * a.k_max : nullptr;
  const int cnt = list ? max(0, min(a.sel_count[gb.bg], a.k_max)) : U;
  const int slots = pg ? cnt * d.P : cnt;
  const float* row = a.logits + ((int64_t)b * d.Hq + h) * d.max_seq;
  const int32_t* bt = a.block_table + (int64_t)b * d.max_pages;
  const int lp = __builtin_ctz(d.P);  // P is a power of two (16 or 64)

  // Slot i of the kept set is token i of the list, or row i % P of its page
  // i / P.  unit_of(i) is the slot's list entry (one load, clamped in range,
  // issued for any i >= 0); logit_of(i, u) is its logit, -inf where the
  // attention kernel attends nothing or past the kept set.  Every load is
  // issued with clamped indices and the result selected afterwards, so a
  // lane's loads overlap instead of draining one slot at a time.
  auto unit_of = [&](int i) -> int {
    const int e = pg ? i >> lp : i;
    return list ? list[min(e, a.k_max - 1)] : e;
  };
  auto logit_of = [&](int i, int u) -> float {
    const int t = pg ? (u << lp) + (i & (d.P - 1)) : u;
    const int tc = t < 0 ? 0 : (t >= n ? max(n - 1, 0) : t);
    const int ph = bt[min(tc >> lp, d.max_pages - 1)];
    const float z = row[tc];
    // bitwise, not short-circuit: a && chain lets the compiler sink the
    // block-table and logit loads under a branch, one slot at a time
    const bool ok = (i < slots) & (u >= 0) & (u < U) & (t < n) & (ph >= 0) &
                    ((int64_t)ph < d.num_pages);
    return ok ? z : -INFINITY;
  };
  // Slots past the registers, in rounds of NT (round k covers slots
  // KPT * NT + k * NT + tid): fn(z) sees every lane's logit of every round in
  // a fixed order (rounds past the end give -inf, and fn is called on every
  // lane, so it may use wave ballots).  Rounds are loaded kTauBatch at a
  // time, list entries first and logits second, so their loads overlap.
  const int tail_rounds = slots > KPT * NT ? (slots - KPT * NT + NT - 1) / NT : 0;
  auto for_tail = [&](auto&& fn) {
    for (int k0 = 0; k0 < tail_rounds; k0 += kTauBatch) {
      int uu[kTauBatch];
      float zz[kTauBatch];
#pragma unroll
      for (int t = 0; t < kTauBatch; ++t) uu[t] = unit_of(KPT * NT + (k0 + t) * NT + tid);
#pragma unroll
      for (int t = 0; t < kTauBatch; ++t) zz[t] = logit_of(KPT * NT + (k0 + t) * NT + tid, uu[t]);
#pragma unroll
      for (int t = 0; t < kTauBatch; ++t) fn(zz[t]);
    }
  };

  float lg[KPT];
  float mx = -INFINITY;
  {
    int uu[KPT];
#pragma unroll
    for (int r = 0; r < KPT; ++r) uu[r] = unit_of(r * NT + tid);
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
      lg[r] = logit_of(r * NT + tid, uu[r]);
      mx = fmaxf(mx, lg[r]);
    }
  }
  for_tail([&](float z) { mx = fmaxf(mx, z); });
  mx = wave_max_dpp(mx);
  if (lane == 0) s_max[wave] = mx;
  __syncthreads();
  mx = -INFINITY;
#pragma unroll
  for (int w = 0; w < NW; ++w) mx = fmaxf(mx, s_max[w]);
  float* out = a.tau + (int64_t)b * d.Hq + h;
  if (mx == -INFINITY) {  // nothing attended: every weight is 0
    if (tid == 0) *out = INFINITY;
    return;
  }

  const float am1 = a.alpha_m1, beta = a.beta;
  const float lo = am1 * mx - 1.f;  // g(lo) >= 0: the largest term alone is ~1
  auto is_cand = [&](float z) { return fmaf(am1, z, -lo) > 0.f; };  // false for -inf

  // Candidates per wave, in slot order: registers r = 0..KPT-1, then the
  // tail rounds, lanes in order within each.
  const uint64_t below = (1ull << lane) - 1ull;
  int wc = 0;
#pragma unroll
  for (int r = 0; r < KPT; ++r) wc += __popcll(__ballot(is_cand(lg[r])));
  for_tail([&](float z) { wc += __popcll(__ballot(is_cand(z))); });
  if (lane == 0) s_cnt[wave] = wc;
  __syncthreads();
  int base = 0, total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    base += w < wave ? s_cnt[w] : 0;
    total += s_cnt[w];
  }

  auto accum = [&](float z, float tau, float& s0, float& s1) {
    const float t = fmaf(am1, z, -tau);
    const float w = entmax_weight(t, beta);
    s0 += w;
    s1 += t > 0.f ? (beta == 2.f ? t : (beta == 1.f ? 1.f : w / t)) : 0.f;
  };
  // Newton step from the sums; returns false when the iteration ends.
  const float e_sub = 1.f - am1;  // S0^(1 - 1/beta) = S0^(2 - alpha)
  auto step = [&](float s0, float s1, float& tau) -> bool {
    if (!(s0 > 1.f)) return false;  // at the root, up to rounding
    const float sub = beta == 1.f ? 1.f : (beta == 2.f ? sqrtf(s0) : exp2f(e_sub * log2f(s0)));
    const float nt = tau + (s0 - sub) / s1;
    if (!(nt > tau)) return false;  // the step no longer moves tau
    tau = nt;
    return true;
  };

  float tau = lo;
  if (total <= kTauCap) {
    int pos = base;
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
      const bool c = is_cand(lg[r]);
      const uint64_t m = __ballot(c);
      if (c) s_c[pos + __popcll(m & below)] = lg[r];
      pos += __popcll(m);
    }
    for_tail([&](float z) {
      const bool c = is_cand(z);
      const uint64_t m = __ballot(c);
      if (c) s_c[pos + __popcll(m & below)] = z;
      pos += __popcll(m);
    });
    __syncthreads();
    if (wave != 0) return;
    for (int it = 0; it < 64; ++it) {
      float s0 = 0.f, s1 = 0.f;
      for (int j = lane; j < total; j += 64) accum(s_c[j], tau, s0, s1);
      s0 = wave_sum_dpp(s0);
      s1 = wave_sum_dpp(s1);
      if (!step(s0, s1, tau)) break;
    }
  } else {
    for (int it = 0; it < 64; ++it) {
      float s0 = 0.f, s1 = 0.f;
#pragma unroll
      for (int r = 0; r < KPT; ++r) accum(lg[r], tau, s0, s1);
      for_tail([&](float z) { accum(z, tau, s0, s1); });
      s0 = wave_sum_dpp(s0);
      s1 = wave_sum_dpp(s1);
      const int par = it & 1;
      if (lane == 0) { s_red[par][0][wave] = s0; s_red[par][1][wave] = s1; }
      __syncthreads();
      s0 = 0.f; s1 = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) { s0 += s_red[par][0][w]; s1 += s_red[par][1][w]; }
      if (!step(s0, s1, tau)) break;
    }
  }
  if (tid == 0) *out = tau;
}

hipError_t launch_entmax_tau(const TauArgs& a, hipStream_t st) {
  const Dims& d = a.d;
  if (!(a.alpha_m1 > 0.f && a.alpha_m1 <= 1.f) || !(a.beta >= 1.f)) return hipErrorInvalidValue;
  if (a.sel_idx && (a.k_max < 1 || !a.sel_count)) return hipErrorInvalidValue;
  if (d.P != 16 && d.P != 64) return hipErrorInvalidValue;
  entmax_tau_kernel<<<dim3(d.B * d.Hq), kTauThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace sdkv
