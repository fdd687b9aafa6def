// Stage 1b with a dropped-mass budget, spread over many blocks per (sequence
// b, KV head g): the same rule as the one-block kernel (budget.hip) -- the
// shortest prefix of the top-k order (decreasing group score, equal scores to
// the lower id) that leaves at most max_dropped of every head's dense softmax
// mass outside, capped at keep_count(U) -- for any number of tokens (the
// softmax normalisers are summed in slice order, so their fp32 rounding can
// differ from the one-block kernel's).  The dropped mass of the discarded
// entries governs the error and is fixed in advance ("Where Activation
// Sparsity and KV-Cache Sparsity Cross in LLM Decoding", cards view, pre-hoc
// sparsity abstract).
//
// A (b, g) is cut into NB <= kQMaxSlices slices of whole 1024-token chunks
// (more, smaller slices measured slower at 128K, fewer larger ones at 32K).
// Block ids are bg + B*Hkv*slice: when B*Hkv is a multiple of the eight XCDs,
// every block of one (b, g) sits on one XCD and the partials exchanged below
// stay in its L2 (any other count is correct, only less local).
//   bm_norm    per slice: each head's largest logit and the sum of the
//              exponentials below it; the min / max order key of the group
//              scores; clears pass 0's histogram;
//   bm_hist    per slice: 256-bin histograms of the keys inside the interval,
//              the count and each head's mass p_h(t) = e^(s - m_h) / Z_h as
//              2^40 fixed-point integers, built in LDS, then added into the
//              (b, g)'s histogram of the pass with global atomics (integer
//              sums do not depend on the order of the atomics, so the result
//              does not depend on timing).  Before pass 0 each block
//              combines the slice partials (the softmax normalisers and the
//              key interval); before pass p > 0 it narrows the interval from
//              pass p - 1's sums: the first bin from the top whose inclusion
//              brings every head within the target, as in the one-block
//              kernel.  Pass p clears pass p + 1's histogram;
//   bm_ties    one block per (b, g): narrows after the last pass; when the
//              interval is one key value, takes its tokens in id order until
//              the target holds; writes the count;
// then the many-block top-k (select_multi.hip) keeps that many units.
#include "topk.h"

namespace sdkv {

namespace {

constexpr int kQT = 256;                 // threads of a slice block
constexpr int kQW = kQT / 64;
constexpr int kQK = 4;                   // tokens per thread per chunk
constexpr int kQChunk = kQT * kQK;       // 1024 tokens
constexpr int kQMaxSlices = 64;          // slices per (b, g)
constexpr int kQBins = 256;
constexpr int kQMaxG = 8;
constexpr int kQPasses = 4;              // 8-bit bins cover any 32-bit interval
constexpr int kTT = 1024;                // tie scan threads
constexpr int kTW = kTT / 64;
constexpr int kTK = 8;                   // ids per thread per tie chunk
constexpr float kQFix = 1099511627776.0f;  // 2^40

typedef unsigned long long u64;

struct QState {
  uint32_t lo, hi;      // the key interval holding the boundary
  uint32_t c_above;     // units above the interval
  uint32_t done;        // no further histogram pass
  int32_t kstar;        // > 0 once the count is known
  int32_t kcap;         // min(keep_count(U), k_max); 0 for an empty sequence
  int32_t pad0, pad1;
  float m[kQMaxG], invz[kQMaxG];
  u64 tot[kQMaxG];      // every unit's mass per head
  u64 above[kQMaxG];    // mass of the units above the interval
};

struct QArgs {
  BudgetArgs a;
  int slice, NB;        // tokens per slice (a multiple of kQChunk); slices per (b, g)
  float2* part;         // [BG][NB][kQMaxG] (largest logit, sum of exponentials)
  uint32_t* mm;         // [BG][NB][2] min / max order key
  QState* st;           // [kQPasses][BG]: the state pass p runs with
  u64* hist;            // [kQPasses][BG][1 + G][kQBins]: counts, then each head's
                        // mass, summed over the slices
  int32_t* kk;          // [BG] the count
};

__device__ __forceinline__ int tokens_of(const BudgetArgs& a, int b) {
  return min(clamp_len(a.seq_lens[b], a.d.max_seq), a.U_max);
}

__device__ __forceinline__ u64 target_of(const BudgetArgs& a) {
  return (u64)(fminf(fmaxf(a.max_dropped, 0.f), 1.f) * kQFix);
}

// The fixed-point mass of a logit s under the normaliser (m, 1 / Z); the
// one-block kernel forms it the same way.
__device__ __forceinline__ u64 fixed_weight(float s, float m, float invz) {
  const float w = exp2f((s - m) * kLog2e) * invz;
  return (u64)(fminf(w, 1.f) * kQFix);
}

// (m, z) <- the pair for the union of two sets, z = sum of e^(s - m).  The
// result does not depend on the argument order (max and a two-term sum).
__device__ __forceinline__ void lse_combine(float& m, float& z, float m2, float z2) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;  // both empty
  z = z * exp2f((m - mn) * kLog2e) + z2 * exp2f((m2 - mn) * kLog2e);
  m = mn;
}

__device__ __forceinline__ void wave_lse(float& m, float& z) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) lse_combine(m, z, __shfl_xor(m, o), __shfl_xor(z, o));
}

__device__ __forceinline__ uint32_t wave_umin32(uint32_t x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = min(x, (uint32_t)__shfl_xor((int)x, o));
  return x;
}
__device__ __forceinline__ uint32_t wave_umax32(uint32_t x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = max(x, (uint32_t)__shfl_xor((int)x, o));
  return x;
}

// Clears this block's share of the (b, g)'s histogram of pass p: the NB
// blocks of the (b, g) share it (block j takes rows j kQT + tid, stepping by
// NB kQT), so every entry is cleared whether or not the block has tokens.
__device__ __forceinline__ void clear_pass_share(const QArgs& q, int bg, int j, int p) {
  const int BG = q.a.d.B * q.a.d.Hkv;
  const int HS = (1 + q.a.d.G) * kQBins;
  u64* hz = q.hist + ((int64_t)p * BG + bg) * HS;
  for (int i = j * kQT + (int)threadIdx.x; i < HS; i += q.NB * kQT) hz[i] = 0ull;
}

// G as a template parameter: every head's loads of a chunk are issued
// before any of them is reduced.
template <int G>
__global__ __launch_bounds__(kQT) void bm_norm_kernel(QArgs q) {
  __shared__ float2 red[kQW][kQMaxG];
  __shared__ uint32_t rmn[kQW], rmx[kQW];
  const BudgetArgs& a = q.a;
  const GroupBlock gb = group_block(a.d.B * a.d.Hkv);
  const int b = gb.bg / a.d.Hkv, g = gb.bg % a.d.Hkv;
  const int U = tokens_of(a, b);
  const int s0 = gb.j * q.slice;
  clear_pass_share(q, gb.bg, gb.j, 0);
  if (s0 >= U) return;  // pass 0 reads only slices holding tokens
  const int s1 = min(s0 + q.slice, U);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* sc = a.scores + (int64_t)gb.bg * a.U_max;
  const float* lg = a.logits + ((int64_t)b * a.d.Hq + (int64_t)g * G) * a.d.max_seq;
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
  float m[G], z[G];
#pragma unroll
  for (int h = 0; h < G; ++h) { m[h] = -INFINITY; z[h] = 0.f; }
  for (int c0 = s0; c0 < s1; c0 += kQChunk) {
    uint32_t key[kQK];
    float x[G][kQK];
#pragma unroll
    for (int i = 0; i < kQK; ++i) {
      const int t = min(c0 + tid + kQT * i, a.U_max - 1);
      key[i] = order_key(sc[t]);
#pragma unroll
      for (int h = 0; h < G; ++h) x[h][i] = lg[(int64_t)h * a.d.max_seq + t];
    }
#pragma unroll
    for (int i = 0; i < kQK; ++i)
      if (c0 + tid + kQT * i < s1) { mn = min(mn, key[i]); mx = max(mx, key[i]); }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float cm = -INFINITY;
#pragma unroll
      for (int i = 0; i < kQK; ++i)
        if (c0 + tid + kQT * i < s1) cm = fmaxf(cm, x[h][i]);
      float cz = 0.f;
#pragma unroll
      for (int i = 0; i < kQK; ++i)
        if (c0 + tid + kQT * i < s1) cz += exp2f((x[h][i] - cm) * kLog2e);
      lse_combine(m[h], z[h], cm, cz);
    }
  }
  mn = wave_umin32(mn);
  mx = wave_umax32(mx);
#pragma unroll
  for (int h = 0; h < G; ++h) {
    wave_lse(m[h], z[h]);
    if (lane == 0) red[wave][h] = make_float2(m[h], z[h]);
  }
  if (lane == 0) { rmn[wave] = mn; rmx[wave] = mx; }
  __syncthreads();
  const int64_t slot = (int64_t)gb.bg * q.NB + gb.j;
  if (tid < G) {
    float pm = red[0][tid].x, pz = red[0][tid].y;
    for (int w = 1; w < kQW; ++w) lse_combine(pm, pz, red[w][tid].x, red[w][tid].y);
    q.part[slot * kQMaxG + tid] = make_float2(pm, pz);
  }
  if (tid == 0) {
    for (int w = 1; w < kQW; ++w) { mn = min(mn, rmn[w]); mx = max(mx, rmx[w]); }
    mn = min(mn, rmn[0]);
    mx = max(mx, rmx[0]);
    q.mm[slot * 2] = mn;
    q.mm[slot * 2 + 1] = mx;
  }
}

// Pass 0's state of a (b, g) into S (every thread of a kQT-thread block
// calls it; S is final after it returns): the softmax normalisers (slice
// partials combined across lanes and waves in a fixed order), the key
// interval [min, max], the cap.
__device__ void initial_state(const QArgs& q, int bg, int U, QState& S) {
  __shared__ float2 red[kQW][kQMaxG];
  __shared__ uint32_t rmn[kQW], rmx[kQW];
  const BudgetArgs& a = q.a;
  const int G = a.d.G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nbv = (U + q.slice - 1) / q.slice;
  // thread t holds slice t (NB <= kQMaxSlices <= kQT): every load is issued
  // before any is combined
  static_assert(kQMaxSlices <= kQT, "one slice per thread");
  const bool have = tid < nbv;
  const int64_t slot = (int64_t)bg * q.NB + (have ? tid : 0);
  uint32_t mn = q.mm[slot * 2], mx = q.mm[slot * 2 + 1];
  float2 pz[kQMaxG];
#pragma unroll
  for (int h = 0; h < kQMaxG; ++h) pz[h] = q.part[slot * kQMaxG + h];
  if (!have) { mn = 0xFFFFFFFFu; mx = 0u; }
  mn = wave_umin32(mn);
  mx = wave_umax32(mx);
  if (lane == 0) { rmn[wave] = mn; rmx[wave] = mx; }
#pragma unroll
  for (int h = 0; h < kQMaxG; ++h) {
    if (h >= G) break;
    float m = have ? pz[h].x : -INFINITY, z = have ? pz[h].y : 0.f;
    wave_lse(m, z);
    if (lane == 0) red[wave][h] = make_float2(m, z);
  }
  __syncthreads();
  if (tid == 0) {
    QState s{};
    s.lo = rmn[0];
    s.hi = rmx[0];
    for (int w = 1; w < kQW; ++w) { s.lo = min(s.lo, rmn[w]); s.hi = max(s.hi, rmx[w]); }
    s.kcap = U > 0 ? min(keep_count_dev(U, a.R_ppm), a.k_max) : 0;
    s.done = s.kcap == 0 ? 1u : 0u;
    for (int h = 0; h < G; ++h) {
      float m = red[0][h].x, z = red[0][h].y;
      for (int w = 1; w < kQW; ++w) lse_combine(m, z, red[w][h].x, red[w][h].y);
      s.m[h] = m;
      s.invz[h] = 1.f / z;
    }
    S = s;
  }
  __syncthreads();
}

// After histogram pass p of a (b, g) (rows: its summed histogram in LDS,
// counts then each head's mass; S: the state the pass ran with, in LDS): the
// next state, also written to *gs unless gs is NULL.  Every thread of the
// block calls it; S is final after a barrier.
__device__ void narrow_after(const BudgetArgs& a, QState& S, const u64* rows, int p,
                             QState* gs) {
  const int G = a.d.G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const u64 target = target_of(a);
  if (p == 0) {
    // every unit is inside the first interval: the totals
    if (tid < G) {
      u64 s = 0ull;
      for (int i = 0; i < kQBins; ++i) s += rows[(1 + tid) * kQBins + i];
      S.tot[tid] = s;
    }
    __syncthreads();
    // keeping no unit already meets the target: one unit is kept
    bool met = true;
    for (int h = 0; h < G; ++h) met = met && S.tot[h] <= target;
    if (met) {
      if (tid == 0) {
        S.kstar = 1;
        S.done = 1u;
        if (gs) *gs = S;
      }
      return;
    }
  }
  if (S.lo == S.hi) {  // one key value: the tie scan decides
    if (tid == 0) {
      S.done = 1u;
      if (gs) *gs = S;
    }
    return;
  }
  if (wave == 0) {
    const uint32_t lo = S.lo, hi = S.hi, shift = bin_shift(lo, hi);
    // lane l holds bins 255 - 4l - j (j < 4): descending order.  ok[j]:
    // keeping everything from bin 255 - 4l - j up meets the target for
    // every head
    bool ok[4] = {true, true, true, true};
    for (int h = 0; h < G; ++h) {
      const u64* mass = rows + (1 + h) * kQBins;
      u64 mb[4], s = 0ull;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        mb[j] = mass[255 - 4 * lane - j];
        s += mb[j];
      }
      u64 run = S.above[h] + (wave_incl_scan<u64>(s) - s);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        run += mb[j];
        if (S.tot[h] > run + target) ok[j] = false;
      }
    }
    int hit = -1;
#pragma unroll
    for (int j = 3; j >= 0; --j)
      if (ok[j]) hit = j;
    const uint64_t hits = __ballot(hit >= 0);
    // keeping the whole interval always meets the target (the lowest bin is
    // a guard); some head is above the target with the units above the
    // interval alone, so the chosen bin holds units
    const int fl = hits ? (int)__builtin_ctzll(hits) : 63;
    const int fj = __shfl(hit >= 0 ? hit : 3, fl, 64);
    const uint32_t bin = (uint32_t)(255 - 4 * fl - fj);
    uint32_t c_up = 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (lane < fl || (lane == fl && j < fj)) c_up += (uint32_t)rows[255 - 4 * lane - j];
    c_up = wave_sum(c_up);
    for (int h = 0; h < G; ++h) {
      const u64* mass = rows + (1 + h) * kQBins;
      u64 m_up = 0ull;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (lane < fl || (lane == fl && j < fj)) m_up += mass[255 - 4 * lane - j];
      m_up = wave_incl_scan<u64>(m_up);
      if (lane == 63) S.above[h] += m_up;
    }
    if (lane == 0) {
      const uint32_t nlo = lo + (bin << shift);
      const uint64_t top = (uint64_t)nlo + ((1ull << shift) - 1ull);
      S.lo = nlo;
      S.hi = (uint32_t)(top < (uint64_t)hi ? top : (uint64_t)hi);
      S.c_above += c_up;
      if (rows[bin] == 1ull) S.kstar = (int)(S.c_above + 1u);  // a bin of one unit
      S.done = (S.kstar > 0 || S.lo == S.hi) ? 1u : 0u;
    }
  }
  __syncthreads();
  if (tid == 0 && gs) *gs = S;
}

// Histogram pass p over one slice, added into the (b, g)'s sums.  Every
// block first derives the pass's state itself -- for p = 0 from the slice
// partials, for p > 0 by narrowing from pass p - 1's sums -- with the same
// steps on the same inputs in every block, so they agree; slice 0 records it
// in st[p].  This saves a launch per pass.
__global__ __launch_bounds__(kQT) void bm_hist_kernel(QArgs q, int p) {
  __shared__ u64 h[(1 + kQMaxG) * kQBins];
  __shared__ QState S;
  const BudgetArgs& a = q.a;
  const int BG = a.d.B * a.d.Hkv;
  const GroupBlock gb = group_block(BG);
  const int b = gb.bg / a.d.Hkv, g = gb.bg % a.d.Hkv, G = a.d.G;
  const int U = tokens_of(a, b);
  const int s0 = gb.j * q.slice;
  if (p + 1 < kQPasses) clear_pass_share(q, gb.bg, gb.j, p + 1);
  if (s0 >= U) return;
  const int tid = threadIdx.x;
  const int HS = (1 + G) * kQBins;
  if (p == 0) {
    // every block combines the slice partials itself; slice 0 records them
    initial_state(q, gb.bg, U, S);
    if (gb.j == 0 && tid == 0) q.st[gb.bg] = S;
  } else {
    if (tid == 0) S = q.st[(int64_t)(p - 1) * BG + gb.bg];
    const u64* prev = q.hist + ((int64_t)(p - 1) * BG + gb.bg) * HS;
    for (int i = tid; i < HS; i += kQT) h[i] = prev[i];
    __syncthreads();
  }
  if (p > 0) {
    QState* rec = gb.j == 0 ? q.st + (int64_t)p * BG + gb.bg : nullptr;
    if (!S.done) {
      narrow_after(a, S, h, p - 1, rec);
      __syncthreads();
    } else if (rec && tid == 0) {
      *rec = S;
    }
  }
  if (S.done) return;  // the same state in every block of the (b, g)
  const uint32_t lo = S.lo, hi = S.hi, shift = bin_shift(lo, hi);
  float m[kQMaxG], invz[kQMaxG];
#pragma unroll
  for (int i = 0; i < kQMaxG; ++i) {
    m[i] = S.m[i];
    invz[i] = S.invz[i];
  }
  __syncthreads();  // h is cleared below
  for (int i = tid; i < HS; i += kQT) h[i] = 0ull;
  __syncthreads();
  const int s1 = min(s0 + q.slice, U);
  const float* sc = a.scores + (int64_t)gb.bg * a.U_max;
  const float* lg = a.logits + ((int64_t)b * a.d.Hq + (int64_t)g * G) * a.d.max_seq;
  for (int c0 = s0; c0 < s1; c0 += kQChunk) {
    uint32_t key[kQK];
#pragma unroll
    for (int i = 0; i < kQK; ++i) key[i] = order_key(sc[min(c0 + tid + kQT * i, a.U_max - 1)]);
#pragma unroll
    for (int i = 0; i < kQK; ++i) {
      const int t = c0 + tid + kQT * i;
      if (t >= s1 || key[i] < lo || key[i] > hi) continue;
      const uint32_t bin = (key[i] - lo) >> shift;
      atomicAdd(&h[bin], 1ull);
#pragma unroll
      for (int hh = 0; hh < kQMaxG; ++hh) {
        if (hh >= G) break;
        atomicAdd(&h[(1 + hh) * kQBins + bin],
                  fixed_weight(lg[(int64_t)hh * a.d.max_seq + t], m[hh], invz[hh]));
      }
    }
  }
  __syncthreads();
  u64* out = q.hist + ((int64_t)p * BG + gb.bg) * HS;
  for (int i = tid; i < HS; i += kQT) {
    const u64 v = h[i];
    if (v != 0ull) atomicAdd(&out[i], v);
  }
}

__global__ __launch_bounds__(kTT) void bm_ties_kernel(QArgs q) {
  __shared__ QState S;
  __shared__ u64 rows[(1 + kQMaxG) * kQBins];
  __shared__ uint64_t tie[kTK * kTW];
  __shared__ int found_s;
  const BudgetArgs& a = q.a;
  const int BG = a.d.B * a.d.Hkv;
  const int bg = blockIdx.x, b = bg / a.d.Hkv, g = bg % a.d.Hkv, G = a.d.G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // an empty sequence has no slice block, so no recorded state: nothing kept
  const int U = tokens_of(a, b);
  if (U == 0) {
    if (tid == 0) q.kk[bg] = 0;
    return;
  }
  // the state after the last pass
  const int HS = (1 + G) * kQBins;
  if (tid == 0) {
    S = q.st[(int64_t)(kQPasses - 1) * BG + bg];
    found_s = 0;
  }
  const u64* last = q.hist + ((int64_t)(kQPasses - 1) * BG + bg) * HS;
  for (int i = tid; i < HS; i += kTT) rows[i] = last[i];
  __syncthreads();
  if (!S.done) {
    narrow_after(a, S, rows, kQPasses - 1, nullptr);
    __syncthreads();
  }
  if (S.kstar > 0) {
    if (tid == 0) q.kk[bg] = max(1, min(S.kstar, S.kcap));
    return;
  }
  // the units whose key is the interval's single value T, in id order
  const uint32_t T = S.lo;
  const u64 target = target_of(a);
  const float* sc = a.scores + (int64_t)bg * a.U_max;
  const float* lg = a.logits + ((int64_t)b * a.d.Hq + (int64_t)g * G) * a.d.max_seq;
  u64 acc[kQMaxG];  // wave 0: mass kept so far per head
#pragma unroll
  for (int h = 0; h < kQMaxG; ++h) acc[h] = S.above[h];
  uint32_t taken = 0u;
  for (int c0 = 0; c0 < U; c0 += kTT * kTK) {
    // word i * kTW + w covers ids c0 + 64 (i * kTW + w) + lane
#pragma unroll
    for (int i = 0; i < kTK; ++i) {
      const int t = c0 + kTT * i + tid;
      const uint64_t w = __ballot(t < U && order_key(sc[min(t, a.U_max - 1)]) == T);
      if (lane == 0) tie[i * kTW + wave] = w;
    }
    __syncthreads();
    if (wave == 0) {
      for (int e = 0; e < kTK * kTW; ++e) {
        const uint64_t word = tie[e];
        if (word == 0ull) continue;
        const int u = c0 + 64 * e + lane;
        const bool mine = (word >> lane) & 1ull;
        bool ok = true;
        u64 tot_word[kQMaxG];
#pragma unroll
        for (int h = 0; h < kQMaxG; ++h) {
          const u64 w = (h < G && mine)
                            ? fixed_weight(lg[(int64_t)h * a.d.max_seq + u], S.m[h], S.invz[h])
                            : 0ull;
          const u64 incl = wave_incl_scan<u64>(w);
          tot_word[h] = __shfl(incl, 63, 64);
          if (h < G && S.tot[h] > acc[h] + incl + target) ok = false;
        }
        const uint64_t sat = __ballot(mine && ok);
        if (sat) {
          const int l = (int)__builtin_ctzll(sat);
          taken += (uint32_t)__popcll(word & ((2ull << l) - 1ull));
          if (lane == 0) found_s = 1;
          break;
        }
        taken += (uint32_t)__popcll(word);
#pragma unroll
        for (int h = 0; h < kQMaxG; ++h) acc[h] += tot_word[h];
      }
    }
    __syncthreads();
    if (found_s) break;
  }
  // every tie taken always meets the target
  if (tid == 0) q.kk[bg] = max(1, min((int)(S.c_above + max(taken, 1u)), S.kcap));
}

struct QLayout {
  int slice, NB;
  size_t part, mm, st, hist, kk, msel, total;
};

QLayout q_layout(const Dims& d, int U_max) {
  QLayout L{};
  const int reps = (U_max + kQChunk * kQMaxSlices - 1) / (kQChunk * kQMaxSlices);
  L.slice = reps * kQChunk;
  L.NB = (U_max + L.slice - 1) / L.slice;
  const int64_t bg = (int64_t)d.B * d.Hkv;
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  size_t off = 0;
  L.part = off; off = up(off + sizeof(float2) * bg * L.NB * kQMaxG);
  L.mm = off;   off = up(off + sizeof(uint32_t) * 2 * bg * L.NB);
  L.st = off;   off = up(off + sizeof(QState) * kQPasses * bg);
  L.hist = off; off = up(off + sizeof(u64) * kQPasses * bg * (1 + d.G) * kQBins);
  L.kk = off;   off = up(off + sizeof(int32_t) * bg);
  L.msel = off; off = up(off + msel_workspace_bytes(d.B, d.Hkv, U_max));
  L.total = off;
  return L;
}

}  // namespace

size_t budget_multi_workspace_bytes(const Dims& d, int U_max) {
  return U_max < 1 ? 0 : q_layout(d, U_max).total;
}

hipError_t launch_select_budget_multi(const BudgetArgs& a, void* ws, hipStream_t st) {
  if (a.U_max < 1 || a.d.G < 1 || a.d.G > kQMaxG || a.k_max < 1 || a.U_max > a.d.max_seq ||
      ws == nullptr)
    return hipErrorInvalidValue;
  const QLayout L = q_layout(a.d, a.U_max);
  char* base = static_cast<char*>(ws);
  QArgs q{};
  q.a = a;
  q.slice = L.slice;
  q.NB = L.NB;
  q.part = reinterpret_cast<float2*>(base + L.part);
  q.mm = reinterpret_cast<uint32_t*>(base + L.mm);
  q.st = reinterpret_cast<QState*>(base + L.st);
  q.hist = reinterpret_cast<u64*>(base + L.hist);
  q.kk = reinterpret_cast<int32_t*>(base + L.kk);
  const int BG = a.d.B * a.d.Hkv;
  const dim3 grid(BG * L.NB);  // block id = bg + B*Hkv*slice
  switch (a.d.G) {
    case 1: bm_norm_kernel<1><<<grid, kQT, 0, st>>>(q); break;
    case 2: bm_norm_kernel<2><<<grid, kQT, 0, st>>>(q); break;
    case 4: bm_norm_kernel<4><<<grid, kQT, 0, st>>>(q); break;
    case 8: bm_norm_kernel<8><<<grid, kQT, 0, st>>>(q); break;
    default: return hipErrorInvalidValue;
  }
  for (int p = 0; p < kQPasses; ++p) bm_hist_kernel<<<grid, kQT, 0, st>>>(q, p);
  bm_ties_kernel<<<BG, kTT, 0, st>>>(q);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  SelectArgs sa{};
  sa.d = a.d;
  sa.unit = kToken;
  sa.seq_lens = a.seq_lens;
  sa.unit_scores = a.scores;
  sa.U_max = a.U_max;
  sa.k_max = a.k_max;
  sa.R_ppm = a.R_ppm;
  sa.sel_idx = a.sel_idx;
  sa.sel_count = a.sel_count;
  return launch_select_multi(sa, q.mm, L.NB, L.slice, base + L.msel, st, q.kk);
}

}  // namespace sdkv
