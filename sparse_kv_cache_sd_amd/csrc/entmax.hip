// alpha-entmax threshold over the kept tokens of every (sequence, query head).
//
// "Where Activation Sparsity and KV-Cache Sparsity Cross in LLM Decoding",
// cards view, EntmaxKV abstract: alpha-entmax attention has exact zeros, so
// sparse decoding over kept candidates that hold its support is exact.  The
// weights over a kept set T are p_t = max((alpha - 1) z_t - tau, 0) ** beta,
// beta = 1 / (alpha - 1), with tau chosen so that they sum to one over T.
//
// f(tau) = sum_t max((alpha - 1) z_t - tau, 0) ** beta - 1 is convex and
// decreasing for 1 < alpha <= 2, with f((alpha - 1) max z - 1) >= 0 and
// f((alpha - 1) max z) = -1.  Newton steps from the left end stay left of
// the root (the tangent of a convex decreasing function lies below it), so
// the iteration climbs monotonically; a bracket [lo, hi] with a bisection
// step guards against rounding.  It stops when a step no longer moves tau
// (typically 4-10 steps at alpha = 1.5; sparsemax ends exactly).
//
// One 1024-thread block per (sequence, query head); block id
// bg + B * H_kv * (h mod G) puts the G heads of a KV head on the XCD that
// runs the attention blocks of that KV head.  The first 32768 kept tokens'
// logits stay in registers (32 per thread) across the iteration; beyond that
// they are re-read each step.  Sums run in a fixed order, so tau does not
// depend on timing.
#include "device.h"

namespace sdkv {

constexpr int kTauThreads = 1024;
constexpr int kTauKeys = 32;

__global__ __launch_bounds__(kTauThreads) void entmax_tau_kernel(TauArgs a) {
  constexpr int NT = kTauThreads, NW = NT / 64, KPT = kTauKeys;
  __shared__ float s_red[2][2][NW];
  __shared__ float s_max[NW];
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

  // Logit of kept slot i (token i of the list, or row i % P of its page i / P),
  // -inf where the attention kernel attends nothing.  Loads are issued with
  // clamped indices and the result is selected afterwards.
  auto slot_logit = [&](int i) -> float {
    const int e = pg ? i / d.P : i;
    const int u = list ? list[min(e, a.k_max - 1)] : e;
    const int t = pg ? u * d.P + (i - e * d.P) : u;
    const int tc = t < 0 ? 0 : (t >= n ? max(n - 1, 0) : t);
    const int ph = bt[min(tc / d.P, d.max_pages - 1)];
    const float z = row[tc];
    const bool ok = u >= 0 && u < U && t < n && ph >= 0 && ph < d.num_pages;
    return ok ? z : -INFINITY;
  };

  float lg[KPT];
  float mx = -INFINITY;
#pragma unroll
  for (int r = 0; r < KPT; ++r) {
    const int i = r * NT + tid;
    lg[r] = i < slots ? slot_logit(i) : -INFINITY;
    mx = fmaxf(mx, lg[r]);
  }
  for (int i = KPT * NT + tid; i < slots; i += NT) mx = fmaxf(mx, slot_logit(i));
  mx = wave_max(mx);
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
  // s0 = sum of weights, s1 = sum of weight / t (= -f'(tau) / beta)
  auto accum = [&](float z, float tau, float& s0, float& s1) {
    const float t = fmaf(am1, z, -tau);
    const float w = entmax_weight(t, beta);
    s0 += w;
    s1 += t > 0.f ? (beta == 2.f ? t : (beta == 1.f ? 1.f : w / t)) : 0.f;
  };
  const float top = am1 * mx;
  float lo = top - 1.f, hi = top, tau = lo;
  for (int it = 0; it < 64; ++it) {
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int r = 0; r < KPT; ++r) accum(lg[r], tau, s0, s1);
    for (int i = KPT * NT + tid; i < slots; i += NT) accum(slot_logit(i), tau, s0, s1);
    s0 = wave_sum(s0);
    s1 = wave_sum(s1);
    const int par = it & 1;
    if (lane == 0) { s_red[par][0][wave] = s0; s_red[par][1][wave] = s1; }
    __syncthreads();
    s0 = 0.f; s1 = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) { s0 += s_red[par][0][w]; s1 += s_red[par][1][w]; }
    const float f = s0 - 1.f;
    if (f >= 0.f) lo = tau; else hi = tau;
    float nt = tau + f / (beta * s1);
    if (f == 0.f || nt == tau) break;
    if (!(nt > lo && nt < hi)) nt = 0.5f * (lo + hi);
    if (nt == tau) break;
    tau = nt;
  }
  if (tid == 0) *out = tau;
}

hipError_t launch_entmax_tau(const TauArgs& a, hipStream_t st) {
  const Dims& d = a.d;
  if (!(a.alpha_m1 > 0.f && a.alpha_m1 <= 1.f) || !(a.beta >= 1.f)) return hipErrorInvalidValue;
  if (a.sel_idx && (a.k_max < 1 || !a.sel_count)) return hipErrorInvalidValue;
  entmax_tau_kernel<<<dim3(d.B * d.Hq), kTauThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace sdkv
