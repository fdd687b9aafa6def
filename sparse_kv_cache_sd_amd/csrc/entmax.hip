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
// weigh exactly 0 at every step: only the others ("candidates") take part,
// and summing a superset of them changes nothing.
//
// Up to kTauChunk (16384) kept slots per head, one 1024-thread block per
// (sequence, query head) holds the logits in registers (16 per thread),
// finds their max, compacts the candidates into LDS in slot order (wave
// ballots and prefix offsets) and lets one wave run the Newton steps with
// wave-level sums only (the values in registers up to 1024 of them, else in
// LDS; the per-value arithmetic compiled for beta = 2, beta = 1 or any
// other beta).  With more slots, chunks of kTauChunk slots go to
// blocks of their own, which leave their max and the slots within
// 1 / (alpha - 1) of it (a superset of the candidates, since a chunk's max
// never exceeds the head's) in the workspace; a merge block per head keeps
// those within reach of the head's max, in chunk order, and iterates as
// above, in a fixed order.  If the candidates do not fit (very flat logits),
// the whole block iterates over every kept logit, re-read each step.  Block ids keep bg =
// (sequence, KV head) fastest, so all blocks of a KV head share the XCD of
// its attention blocks.  Sums run in a fixed order, so tau does not depend
// on timing.
#include <type_traits>

#include "device.h"

namespace sdkv {

constexpr int kTauThreads = 1024;
constexpr int kTauKeys = kTauChunk / kTauThreads;  // logits per thread in registers
constexpr int kTauCap = 12288;   // candidates compacted into LDS (48 KB)
static_assert(kTauMaxChunks <= kTauThreads, "the merge reads a chunk per thread");
constexpr int kTauBatch = 8;     // rounds whose loads are issued together
static_assert(kTauKeys * kTauThreads == kTauChunk, "a chunk fills the registers");

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

// The kept slots of one (sequence, query head).  Slot i is token i of the
// list, or row i % P of its page i / P.  unit_of(i) is the slot's list entry
// (one load, clamped in range, issued for any i >= 0); logit_of(i, u) is its
// logit, -inf where the attention kernel attends nothing or past the kept
// set.  Every load is issued with clamped indices and the result selected
// afterwards, so a lane's loads overlap instead of draining one slot at a
// time.
struct Slots {
  const int32_t* list;
  const int32_t* bt;
  const float* row;
  int k_max, n, U, slots, lp, P, max_pages, last;
  int64_t num_pages;
  bool pg, by_slot;

  __device__ Slots(const TauArgs& a, int b, int bg, int h) {
    const Dims& d = a.d;
    n = clamp_len(a.seq_lens[b], d.max_seq);
    pg = a.unit == kPage;
    P = d.P;
    lp = __builtin_ctz(d.P);  // P is a power of two (16 or 64)
    U = pg ? (n + d.P - 1) / d.P : n;
    list = a.sel_idx ? a.sel_idx + (int64_t)bg * a.k_max : nullptr;
    k_max = a.k_max;
    const int cnt = list ? max(0, min(a.sel_count[bg], a.k_max)) : U;
    slots = pg ? cnt * d.P : cnt;
    row = a.logits + ((int64_t)b * d.Hq + h) * d.max_seq;
    bt = a.block_table + (int64_t)b * d.max_pages;
    by_slot = a.logits_slots != 0;
    // the last slot the logits pass wrote: its splits cover the list's k_max
    // entries, or every unit without a list
    last = (list ? (pg ? k_max * d.P : k_max) : d.max_seq) - 1;
    max_pages = d.max_pages;
    num_pages = d.num_pages;
  }
  __device__ __forceinline__ int unit_of(int i) const {
    if (by_slot) return 0;  // not needed
    const int e = pg ? i >> lp : i;
    return list ? list[min(e, k_max - 1)] : e;
  }
  __device__ __forceinline__ float logit_of(int i, int u) const {
    if (by_slot) {  // slot i directly (its writer put -inf where nothing is attended)
      const float z = row[min(max(i, 0), last)];  // a bound known without the count
      return i < slots ? z : -INFINITY;
    }
    const int t = pg ? (u << lp) + (i & (P - 1)) : u;
    const int tc = t < 0 ? 0 : (t >= n ? max(n - 1, 0) : t);
    const int ph = bt[min(tc >> lp, max_pages - 1)];
    const float z = row[tc];
    // bitwise, not short-circuit: a && chain lets the compiler sink the
    // block-table and logit loads under a branch, one slot at a time
    const bool ok = (i < slots) & (u >= 0) & (u < U) & (t < n) & (ph >= 0) &
                    ((int64_t)ph < num_pages);
    return ok ? z : -INFINITY;
  }
  // fn(z) for every slot in [from, to), in rounds of kTauThreads (round k
  // covers slots from + k * NT + tid; slots past `to` give -inf), on every
  // lane, kTauBatch rounds' loads issued together.
  template <typename Fn>
  __device__ __forceinline__ void for_range(int from, int to, Fn&& fn) const {
    constexpr int NT = kTauThreads;
    const int tid = threadIdx.x;
    const int rounds = to > from ? (to - from + NT - 1) / NT : 0;
    for (int k0 = 0; k0 < rounds; k0 += kTauBatch) {
      int uu[kTauBatch];
      float zz[kTauBatch];
#pragma unroll
      for (int t = 0; t < kTauBatch; ++t) uu[t] = unit_of(from + (k0 + t) * NT + tid);
#pragma unroll
      for (int t = 0; t < kTauBatch; ++t) {
        const int i = from + (k0 + t) * NT + tid;
        const float z = logit_of(i, uu[t]);
        zz[t] = i < to ? z : -INFINITY;
      }
#pragma unroll
      for (int t = 0; t < kTauBatch; ++t) fn(zz[t]);
    }
  }
};

// Exponent classes of the weights, fixed per launch: beta = 2 (alpha = 1.5:
// squares), beta = 1 (sparsemax: the positive parts themselves), any other
// beta (exp2 / log2).  The Newton loops are compiled once per class so that
// the per-value work has no branches.
enum BetaKind : int { kBetaAny = 0, kBetaOne = 1, kBetaTwo = 2 };

// The alpha-entmax arithmetic of one head.
struct Newton {
  float am1, beta, e_sub;
  __device__ Newton(const TauArgs& a) : am1(a.alpha_m1), beta(a.beta), e_sub(1.f - a.alpha_m1) {}
  // s0 = sum of weights max(t, 0)^beta, s1 = sum of max(t, 0)^(beta - 1)
  // (= -f'(tau) / beta), t = (alpha - 1) z - tau
  template <int K>
  __device__ __forceinline__ void accum(float z, float tau, float& s0, float& s1) const {
    const float t = fmaf(am1, z, -tau);
    if constexpr (K == kBetaTwo) {
      const float p = fmaxf(t, 0.f);
      s0 += p * p;
      s1 += p;
    } else if constexpr (K == kBetaOne) {
      s0 += fmaxf(t, 0.f);
      s1 += t > 0.f ? 1.f : 0.f;
    } else {
      const float lt = log2f(t);  // used only where t > 0
      s0 += t > 0.f ? exp2f(beta * lt) : 0.f;
      s1 += t > 0.f ? exp2f((beta - 1.f) * lt) : 0.f;
    }
  }
  // Newton step on g from the sums; false when the iteration ends.
  template <int K>
  __device__ __forceinline__ bool step(float s0, float s1, float& tau) const {
    if (!(s0 > 1.f)) return false;  // at the root, up to rounding
    const float sub = K == kBetaOne ? 1.f : (K == kBetaTwo ? sqrtf(s0) : exp2f(e_sub * log2f(s0)));
    const float nt = tau + (s0 - sub) / s1;
    if (!(nt > tau)) return false;  // the step no longer moves tau
    tau = nt;
    return true;
  }
  __device__ __forceinline__ bool cand(float z, float lo) const { return fmaf(am1, z, -lo) > 0.f; }
  // fn(integral_constant<int, K>) for this head's exponent class
  template <typename Fn>
  __device__ __forceinline__ float by_kind(Fn&& fn) const {
    if (beta == 2.f) return fn(std::integral_constant<int, kBetaTwo>{});
    if (beta == 1.f) return fn(std::integral_constant<int, kBetaOne>{});
    return fn(std::integral_constant<int, kBetaAny>{});
  }
};

// Block-wide max of a per-thread value (every thread gets it).
template <int NW>
__device__ __forceinline__ float block_max(float v, float* s_max) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_max_dpp(v);
  if (lane == 0) s_max[wave] = v;
  __syncthreads();
  v = -INFINITY;
#pragma unroll
  for (int w = 0; w < NW; ++w) v = fmaxf(v, s_max[w]);
  return v;
}

// Newton steps by one wave over n values at s_c; returns tau.  Lane l owns
// the values s_c[l + 64 k] and sums them in k order.  Up to 64 R values stay
// in registers (R per lane, -inf past n) for every step.
template <int K, int R>
__device__ __forceinline__ float newton_regs(const Newton& nw, const float* s_c, int n,
                                             float tau) {
  const int lane = threadIdx.x & 63;
  float z[R];
#pragma unroll
  for (int r = 0; r < R; ++r) z[r] = lane + 64 * r < n ? s_c[lane + 64 * r] : -INFINITY;
  for (int it = 0; it < 64; ++it) {
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) nw.accum<K>(z[r], tau, s0, s1);
    s0 = wave_sum_dpp(s0);
    s1 = wave_sum_dpp(s1);
    if (!nw.step<K>(s0, s1, tau)) break;
  }
  return tau;
}

// More values: they stay in LDS.  tau only grows, so a value whose weight is
// zero at one step is zero at every later one: each step keeps, in order and
// in place, only the lane's values still positive, and later steps read
// fewer.  Dropped values add exactly 0 to both sums, so the sums (and tau)
// are those of the full list.  The LDS reads go in batches of eight, issued
// together.  s_c is overwritten.
template <int K>
__device__ __forceinline__ float newton_lds(const Newton& nw, float* s_c, int n, float tau) {
  constexpr int R = 8;
  const int lane = threadIdx.x & 63;
  int m = lane < n ? (n - 1 - lane) / 64 + 1 : 0;  // this lane's values
  for (int it = 0; it < 64; ++it) {
    float s0 = 0.f, s1 = 0.f;
    int keep = 0;
    for (int k = 0; k < m; k += R) {
      // all R reads first (indices clamped to the lane's last value), then
      // the values in order; writes land at or below the values read
      float z[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        z[r] = s_c[lane + 64 * min(k + r, m - 1)];
        if (k + r >= m) z[r] = -INFINITY;
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        nw.accum<K>(z[r], tau, s0, s1);
        if (fmaf(nw.am1, z[r], -tau) > 0.f) s_c[lane + 64 * keep++] = z[r];
      }
    }
    m = keep;
    s0 = wave_sum_dpp(s0);
    s1 = wave_sum_dpp(s1);
    if (!nw.step<K>(s0, s1, tau)) break;
  }
  return tau;
}

// The values' count picks registers (up to 1024) or LDS.
__device__ __forceinline__ float newton_wave(const Newton& nw, float* s_c, int n, float tau) {
  return nw.by_kind([&](auto kind) {
    constexpr int K = decltype(kind)::value;
    if (n <= 64 * 8) return newton_regs<K, 8>(nw, s_c, n, tau);
    if (n <= 64 * 16) return newton_regs<K, 16>(nw, s_c, n, tau);
    return newton_lds<K>(nw, s_c, n, tau);
  });
}

// Newton steps by the whole block over every kept logit, re-read each step
// (the fallback for candidates that do not fit in LDS).
template <int NW>
__device__ __forceinline__ float newton_block(const Newton& nw, const Slots& sl, float tau,
                                              float (*s_red)[2][NW]) {
  return nw.by_kind([&](auto kind) {
    constexpr int K = decltype(kind)::value;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    float t = tau;
    for (int it = 0; it < 64; ++it) {
      float s0 = 0.f, s1 = 0.f;
      sl.for_range(0, sl.slots, [&](float z) { nw.accum<K>(z, t, s0, s1); });
      s0 = wave_sum_dpp(s0);
      s1 = wave_sum_dpp(s1);
      const int par = it & 1;
      if (lane == 0) { s_red[par][0][wave] = s0; s_red[par][1][wave] = s1; }
      __syncthreads();
      s0 = 0.f; s1 = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) { s0 += s_red[par][0][w]; s1 += s_red[par][1][w]; }
      if (!nw.step<K>(s0, s1, t)) break;
    }
    return t;
  });
}

// One block per head, at most kTauChunk kept slots.
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
  const Slots sl(a, b, gb.bg, h);
  const Newton nw(a);

  float lg[KPT];
  float mx = -INFINITY;
  {
    int uu[KPT];
#pragma unroll
    for (int r = 0; r < KPT; ++r) uu[r] = sl.unit_of(r * NT + tid);
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
      lg[r] = sl.logit_of(r * NT + tid, uu[r]);
      mx = fmaxf(mx, lg[r]);
    }
  }
  // (the host sends more slots than the registers hold to the chunk
  // kernels; should it not, the slots past them still count)
  const bool fits = sl.slots <= KPT * NT;
  if (!fits) sl.for_range(KPT * NT, sl.slots, [&](float z) { mx = fmaxf(mx, z); });
  mx = block_max<NW>(mx, s_max);
  float* out = a.tau + (int64_t)b * d.Hq + h;
  if (mx == -INFINITY) {  // nothing attended: every weight is 0
    if (tid == 0) *out = INFINITY;
    return;
  }
  const float lo = nw.am1 * mx - 1.f;  // g(lo) >= 0: the largest term alone is ~1
  if (!fits) {
    const float tau = newton_block<NW>(nw, sl, lo, s_red);
    if (tid == 0) *out = tau;
    return;
  }

  // Candidates per wave, in slot order (register r, then lane).
  const uint64_t below = (1ull << lane) - 1ull;
  int wc = 0;
#pragma unroll
  for (int r = 0; r < KPT; ++r) wc += __popcll(__ballot(nw.cand(lg[r], lo)));
  if (lane == 0) s_cnt[wave] = wc;
  __syncthreads();
  int base = 0, total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    base += w < wave ? s_cnt[w] : 0;
    total += s_cnt[w];
  }
  float tau = lo;
  if (total <= kTauCap) {
    int pos = base;
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
      const bool c = nw.cand(lg[r], lo);
      const uint64_t m = __ballot(c);
      if (c) s_c[pos + __popcll(m & below)] = lg[r];
      pos += __popcll(m);
    }
    __syncthreads();
    if (wave != 0) return;
    tau = newton_wave(nw, s_c, total, tau);
  } else {
    tau = newton_block<NW>(nw, sl, tau, s_red);
  }
  if (tid == 0) *out = tau;
}

// One block per (head, chunk of kTauChunk slots): the chunk's max and its
// slots within 1 / (alpha - 1) of it, in slot order, to the workspace
// (count kTauChunkCap + 1: more than fit, none written).
__global__ __launch_bounds__(kTauThreads) void entmax_chunk_kernel(TauArgs a) {
  constexpr int NT = kTauThreads, NW = NT / 64, KPT = kTauKeys;
  __shared__ float s_max[NW];
  __shared__ int s_cnt[NW];
  const Dims& d = a.d;
  const int BG = d.B * d.Hkv;
  const GroupBlock gb = group_block(BG);  // gb.j = head in group + G * chunk
  const int j = gb.j % d.G, c = gb.j / d.G;
  const int g = gb.bg % d.Hkv, b = gb.bg / d.Hkv, h = g * d.G + j;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const Slots sl(a, b, gb.bg, h);
  const Newton nw(a);
  const int64_t hc = ((int64_t)b * d.Hq + h) * a.nch + c;
  const int from = c * kTauChunk;

  float lg[KPT];
  float mx = -INFINITY;
  {
    int uu[KPT];
#pragma unroll
    for (int r = 0; r < KPT; ++r) uu[r] = sl.unit_of(from + r * NT + tid);
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
      lg[r] = sl.logit_of(from + r * NT + tid, uu[r]);
      mx = fmaxf(mx, lg[r]);
    }
  }
  mx = block_max<NW>(mx, s_max);
  const float lo = nw.am1 * mx - 1.f;
  const uint64_t below = (1ull << lane) - 1ull;
  int wc = 0;
#pragma unroll
  for (int r = 0; r < KPT; ++r) wc += __popcll(__ballot(nw.cand(lg[r], lo)));
  if (lane == 0) s_cnt[wave] = wc;
  __syncthreads();
  int base = 0, total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    base += w < wave ? s_cnt[w] : 0;
    total += s_cnt[w];
  }
  if (tid == 0) {
    a.cmax[hc] = mx;
    a.ccnt[hc] = total <= kTauChunkCap ? total : kTauChunkCap + 1;
  }
  if (total > kTauChunkCap) return;
  float* dst = a.cand + hc * kTauChunkCap;
  int pos = base;
#pragma unroll
  for (int r = 0; r < KPT; ++r) {
    const bool cnd = nw.cand(lg[r], lo);  // false for -inf (empty chunk)
    const uint64_t m = __ballot(cnd);
    if (cnd) dst[pos + __popcll(m & below)] = lg[r];
    pos += __popcll(m);
  }
}

// One block per head after entmax_chunk_kernel: the head's max over the
// chunks, its candidates gathered from the chunks' lists in chunk order,
// then the Newton steps (one wave), or the block-wide fallback.  Thread c
// reads chunk c's max and count (one round trip for all chunks; nch <=
// kTauMaxChunks); the lists are then read as one concatenated list, in rounds
// of kTauThreads entries.
__global__ __launch_bounds__(kTauThreads) void entmax_merge_kernel(TauArgs a) {
  constexpr int NT = kTauThreads, NW = NT / 64;
  __shared__ float s_c[kTauCap];
  __shared__ float s_red[2][2][NW];
  __shared__ float s_max[NW];
  __shared__ int s_cnt[NW];
  __shared__ int s_off[kTauMaxChunks + 1];  // chunk c's entries start at s_off[c]
  const Dims& d = a.d;
  const GroupBlock gb = group_block(d.B * d.Hkv);
  const int g = gb.bg % d.Hkv, b = gb.bg / d.Hkv, h = g * d.G + gb.j;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const Slots sl(a, b, gb.bg, h);
  const Newton nw(a);
  const int64_t h0 = ((int64_t)b * d.Hq + h) * a.nch;
  // every allocated chunk: entmax_chunk_kernel writes max -inf and count 0
  // for the chunks past the kept slots, so the reads need not wait for the
  // list's count
  const int nch = a.nch;

  const bool mine = tid < nch;
  const float cm = mine ? a.cmax[h0 + tid] : -INFINITY;
  const int cc = mine ? a.ccnt[h0 + tid] : 0;
  const bool over = __syncthreads_or(cc > kTauChunkCap);
  const float mx = block_max<NW>(cm, s_max);
  float* out = a.tau + (int64_t)b * d.Hq + h;
  if (mx == -INFINITY) {  // nothing attended: every weight is 0
    if (tid == 0) *out = INFINITY;
    return;
  }
  const float lo = nw.am1 * mx - 1.f;
  float tau = lo;
  bool full = over;
  if (!over) {
    // exclusive prefix of the chunk counts, in chunk order
    const int incl = wave_incl_scan<int>(cc);
    if (lane == 63) s_cnt[wave] = incl;
    __syncthreads();
    int wbase = 0, raw = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      wbase += w < wave ? s_cnt[w] : 0;
      raw += s_cnt[w];
    }
    if (mine) s_off[tid] = wbase + incl - cc;
    if (tid == 0) s_off[nch] = raw;
    __syncthreads();  // s_cnt is rewritten below
    // the candidates of the head's max, kept in order by block-wide ballot
    // prefix offsets
    const uint64_t below = (1ull << lane) - 1ull;
    int total = 0;
    for (int e0 = 0; e0 < raw; e0 += NT) {
      const int e = e0 + tid;
      float z = -INFINITY;
      if (e < raw) {
        int lo_c = 0, hi_c = nch - 1;  // the chunk holding entry e
        while (lo_c < hi_c) {
          const int mid = (lo_c + hi_c + 1) >> 1;
          if (s_off[mid] <= e) lo_c = mid;
          else hi_c = mid - 1;
        }
        z = a.cand[(h0 + lo_c) * kTauChunkCap + (e - s_off[lo_c])];
      }
      const bool cnd = nw.cand(z, lo);
      const uint64_t m = __ballot(cnd);
      if (lane == 0) s_cnt[wave] = __popcll(m);
      __syncthreads();
      int base = total, add = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        base += w < wave ? s_cnt[w] : 0;
        add += s_cnt[w];
      }
      const int pos = base + __popcll(m & below);
      if (cnd && pos < kTauCap) s_c[pos] = z;
      total += add;
      __syncthreads();  // s_cnt is rewritten next round
    }
    full = total > kTauCap;
    if (!full) {
      if (wave != 0) return;
      tau = newton_wave(nw, s_c, total, tau);
      if (tid == 0) *out = tau;
      return;
    }
  }
  tau = newton_block<NW>(nw, sl, tau, s_red);
  if (tid == 0) *out = tau;
}

hipError_t launch_entmax_tau(const TauArgs& a, hipStream_t st) {
  const Dims& d = a.d;
  if (!(a.alpha_m1 > 0.f && a.alpha_m1 <= 1.f) || !(a.beta >= 1.f)) return hipErrorInvalidValue;
  if (a.sel_idx && (a.k_max < 1 || !a.sel_count)) return hipErrorInvalidValue;
  if (d.P != 16 && d.P != 64) return hipErrorInvalidValue;
  if (a.nch < 0 || (a.nch > 0 && (!a.cand || !a.cmax || !a.ccnt))) return hipErrorInvalidValue;
  if (a.nch > kTauMaxChunks) return hipErrorInvalidValue;  // one chunk per merge thread
  if (a.nch == 0) {
    entmax_tau_kernel<<<dim3(d.B * d.Hq), kTauThreads, 0, st>>>(a);
  } else {
    entmax_chunk_kernel<<<dim3(d.B * d.Hq * a.nch), kTauThreads, 0, st>>>(a);
    entmax_merge_kernel<<<dim3(d.B * d.Hq), kTauThreads, 0, st>>>(a);
  }
  return hipGetLastError();
}

}  // namespace sdkv
