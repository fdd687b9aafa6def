// Exact top-k of one selection instance inside a thread block (used by the
// standalone selection kernel and by the attention kernel, which selects its
// own slice of the kept list).
//
// Keeps the k largest scores, equal scores going to the lower unit id, and
// reports each kept id with its rank in ascending id order (the selected
// block set over which attention runs: "SparDA: Sparse Decoupled Attention
// ..." summary, Section 3.1 and Appendix A).  Keys are held interleaved
// (thread t holds units t, t + NT, t + 2 NT, ...) so that they load with
// coalesced reads.
//
// A float maps to an order-preserving 32-bit key (-0 folded onto +0).  The
// search keeps a key interval [lo, hi] known to hold the k-th largest key and
// the number `need` of keys still to take from it (every key above hi is
// kept).  Each pass splits the interval into 256 equal bins of 2^shift keys,
// counts the keys per bin in LDS, and moves to the bin holding the need-th
// largest.  Starting from the block's [min, max] keeps the bins populated, so
// the LDS counters see little contention.  A pass whose bin is needed whole
// ends the search: every key >= the bin's lower edge is kept.  Otherwise the
// bins shrink to single keys, T = lo is the k-th largest key, and the first
// `need` keys equal to T in index order are kept.  The kept set is then a
// bitmap (one ballot per 64 consecutive units), and a scan of the word counts
// in index order gives every kept id its rank.  All counting is integer, so
// the result does not depend on thread timing.
#pragma once

#include "device.h"

namespace sdkv {

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// k = clamp(ceil(R * U / 1e6), 1, U); R < 0 keeps all U.
__device__ __forceinline__ int keep_count_dev(int U, int R_ppm) {
  if (U <= 0) return 0;
  if (R_ppm < 0) return U;
  const int64_t kk = ((int64_t)R_ppm * U + 999999) / 1000000;
  return (int)(kk < 1 ? 1 : (kk > U ? U : kk));
}

// With many keys per thread the 256 bin counters exist in kHistCopies
// interleaved copies: lane l adds to copy l % kHistCopies, so lanes of one
// wave whose keys share a bin mostly hit different words (LDS atomics to one
// word serialise, and score distributions crowd a few bins).  Rows are 257
// words apart so that the copies of a bin sit in different banks.  Word 256
// of each row is that copy's sink: a key outside the interval adds 0 there
// instead of branching.  The copies are summed into `total` before the bin
// is chosen; all counts are integers, so the result does not depend on the
// order of the adds.  With few keys per thread one copy is used (row 0): the
// extra clearing and summing would cost more than the collisions.
constexpr int kHistCopies = 16;
constexpr int kHistRow = 257;

struct RadixState {
  uint32_t hist[kHistCopies * kHistRow];
  uint32_t total[256];
  uint32_t wa[16], wb[16];
  uint32_t lo, hi, need, whole, shift;
};

// Block-wide min and max of the keys (NW waves); result in st.lo / st.hi.
// (Block sizes are compile-time constants throughout: reading blockDim or
// gridDim can cost a read of the dispatch packet.)
template <int NW>
__device__ __forceinline__ void block_minmax(RadixState& st, uint32_t mn, uint32_t mx) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int nw = NW;
  mn = wave_umin(mn);
  mx = wave_umax(mx);
  if (lane == 0) { st.wa[wave] = mn; st.wb[wave] = mx; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < nw; ++w) { mn = min(mn, st.wa[w]); mx = max(mx, st.wb[w]); }
    st.lo = mn;
    st.hi = mx;
  }
  __syncthreads();
}

// Width of the bins for the interval [lo, hi]: 256 bins cover it.
__device__ __forceinline__ uint32_t bin_shift(uint32_t lo, uint32_t hi) {
  const uint32_t span = hi - lo;
  const int bits = span == 0u ? 0 : 32 - __clz(span);
  return bits > 8 ? bits - 8 : 0;
}

// After a histogram pass (wave 0): find the bin holding the need-th largest
// key of [lo, hi] from the 256 counts, lanes covering bins from the top
// down, and narrow to it.
__device__ __forceinline__ void find_bin(RadixState& st, const uint32_t* counts) {
  const int lane = threadIdx.x & 63;
  const uint32_t need = st.need, lo = st.lo, hi = st.hi, shift = st.shift;
  uint32_t c[4], tot = 0u;
#pragma unroll
  for (int i = 0; i < 4; ++i) { c[i] = counts[255 - 4 * lane - i]; tot += c[i]; }
  uint32_t run = wave_scan_dpp(tot) - tot;  // keys in higher bins
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (run < need && run + c[i] >= need) {
      const uint32_t bin = uint32_t(255 - 4 * lane - i);
      const uint32_t nlo = lo + (bin << shift);
      const uint64_t top = (uint64_t)nlo + ((1ull << shift) - 1ull);
      st.lo = nlo;
      st.hi = (uint32_t)(top < (uint64_t)hi ? top : (uint64_t)hi);
      st.need = need - run;
      st.whole = c[i] == need - run;
    }
    run += c[i];
  }
}

// Exclusive block scan of two counters at once (at most 16 waves).
__device__ __forceinline__ void block_excl_scan2(RadixState& st, uint32_t a, uint32_t b,
                                                 uint32_t* ea, uint32_t* eb) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t ia = wave_scan_dpp(a), ib = wave_scan_dpp(b);
  if (lane == 63) { st.wa[wave] = ia; st.wb[wave] = ib; }
  __syncthreads();
  uint32_t oa = 0u, ob = 0u;
  for (int w = 0; w < wave; ++w) { oa += st.wa[w]; ob += st.wb[w]; }
  *ea = oa + ia - a;
  *eb = ob + ib - b;
  __syncthreads();
}

// The kept set as a bitmap, for keys held interleaved (key[i] of thread t is
// unit t + NT*i, so the ballot of slot i in wave w is the 64-bit word of units
// 64 (i*NW + w) .. +63: words in ascending unit order).  Kept = above T (or
// >= T for a whole bin), plus the first `need` units equal to T in id order,
// plus every unit u < f_lo or u >= f_hi (forced units, for the union of the
// top-k with the first and last units).  On return (after a barrier)
// s_mask[e] holds the kept units of word e and s_base[e] the number of kept
// units in the words before it, so a kept unit's rank in the ascending list
// is s_base[e] + its position among the word's set bits; *s_total (if given)
// is the number of kept units.  One wave trims the ties and scans the word
// counts.
template <int KPT, int NW>
__device__ __forceinline__ void kept_words(uint64_t* s_mask, uint64_t* s_tie, uint32_t* s_base,
                                           const uint32_t (&key)[KPT], int U, uint32_t T,
                                           uint32_t need, bool whole, int f_lo = 0,
                                           int f_hi = 0x7FFFFFFF, uint32_t* s_total = nullptr) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int NT = NW * 64, W = KPT * NW;
  constexpr int PPL = (W + 63) / 64;  // words per scanning lane
  static_assert(PPL <= 8, "at most 512 words");
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int u = (int)threadIdx.x + NT * i;
    const bool v = u < U;
    const uint64_t above =
        __ballot(v && ((whole ? key[i] >= T : key[i] > T) || u < f_lo || u >= f_hi));
    const uint64_t tie = __ballot(v && !whole && key[i] == T);
    if (lane == 0) {
      s_mask[i * NW + wave] = above;
      s_tie[i * NW + wave] = tie;
    }
  }
  __syncthreads();
  if (wave == 0) {
    uint64_t m[PPL], t[PPL];
    uint32_t tc = 0u;
#pragma unroll
    for (int q = 0; q < PPL; ++q) {
      const int e = PPL * lane + q;
      m[q] = e < W ? s_mask[e] : 0ull;
      t[q] = e < W ? s_tie[e] : 0ull;
      tc += __popcll(t[q]);
    }
    uint32_t ties_before = wave_scan_dpp(tc) - tc;
    uint32_t kc = 0u;
#pragma unroll
    for (int q = 0; q < PPL; ++q) {
      const uint32_t c = __popcll(t[q]);
      // max(need - ties_before, 0) as a signed difference: written as an
      // unsigned conditional subtract it became a saturating subtract that
      // the code generator emitted without its clamp.
      const int rem = max((int)need - (int)ties_before, 0);
      const uint32_t keep = min((uint32_t)rem, c);
      uint64_t rest = t[q];  // drop the `keep` lowest tie bits from rest
      for (uint32_t r = 0; r < keep; ++r) rest &= rest - 1ull;
      m[q] |= t[q] ^ rest;
      ties_before += c;
      kc += __popcll(m[q]);
    }
    uint32_t base = wave_scan_dpp(kc) - kc;
#pragma unroll
    for (int q = 0; q < PPL; ++q) {
      const int e = PPL * lane + q;
      if (e < W) {
        s_mask[e] = m[q];
        s_base[e] = base;
      }
      base += __popcll(m[q]);
    }
    if (s_total && lane == 63) *s_total = base;
  }
  __syncthreads();
}

// Calls emit(rank, unit) for every kept unit whose rank lies in [r_lo, r_hi),
// from the bitmap of kept_words.  With few keys per thread each thread ranks
// its own keys (unit t + NT*i is bit `lane` of word i*NW + wave; a wave skips
// a word whose ranks lie outside the range); with many, threads take a word
// each and walk its set bits, skipping words outside the range.
template <int KPT, int NW, typename Emit>
__device__ __forceinline__ void emit_kept(const uint64_t* s_mask, const uint32_t* s_base,
                                          uint32_t r_lo, uint32_t r_hi, Emit&& emit) {
  constexpr int NT = NW * 64;
  if constexpr (KPT < 16) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const uint64_t m = s_mask[i * NW + wave];
      const uint32_t base = s_base[i * NW + wave];
      if (base >= r_hi || base + (uint32_t)__popcll(m) <= r_lo) continue;  // uniform
      const uint32_t pos = base + (uint32_t)__popcll(m & below);
      if (((m >> lane) & 1ull) && pos >= r_lo && pos < r_hi)
        emit((int)pos, (int)threadIdx.x + NT * i);
    }
  } else {
    constexpr int W = KPT * NW;
    for (int e = threadIdx.x; e < W; e += NT) {
      uint64_t m = s_mask[e];
      uint32_t pos = s_base[e];
      if (pos >= r_hi || pos + (uint32_t)__popcll(m) <= r_lo) continue;
      while (m != 0ull) {
        const int bit = __builtin_ctzll(m);
        if (pos >= r_lo && pos < r_hi) emit((int)pos, 64 * e + bit);
        ++pos;
        m &= m - 1ull;
      }
    }
  }
}

template <int KPT, int NW>
struct KeptScratch {
  uint64_t mask[KPT * NW], tie[KPT * NW];
  uint32_t base[KPT * NW];
  uint32_t total;  // kept units
};

// The exact top-k search over keys held in registers, interleaved (key[i] of
// thread t is unit t + NT*i; keys past U are ignored): the final interval in
// lo / need / whole -- every key above it is kept, and need more from it (all
// of it when whole; else it is the single k-th largest key T).
template <int KPT, int NW>
__device__ __forceinline__ void radix_search(RadixState& st, const uint32_t (&key)[KPT], int U,
                                             int k, uint32_t* lo_out, uint32_t* need_out,
                                             bool* whole_out) {
  constexpr int NT = NW * 64;
  const int tid = threadIdx.x;
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
  for (int i = 0; i < KPT; ++i)
    if (tid + NT * i < U) { mn = min(mn, key[i]); mx = max(mx, key[i]); }
  block_minmax<NW>(st, mn, mx);
  if (tid == 0) { st.need = (uint32_t)k; st.whole = 0u; }
  __syncthreads();
  uint32_t lo = st.lo, hi = st.hi;
  bool whole = false;
  while (!whole && lo != hi) {
    const uint32_t shift = bin_shift(lo, hi);
    constexpr int C = KPT >= 16 ? kHistCopies : 1;
    for (int i = tid; i < C * kHistRow; i += NT) st.hist[i] = 0u;
    if (tid == 0) st.shift = shift;
    __syncthreads();
    uint32_t* row = st.hist + (C > 1 ? (tid % C) * kHistRow : 0);
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const bool in = tid + NT * i < U && key[i] >= lo && key[i] <= hi;
      // one copy: a per-lane sink past the row keeps the zero adds apart
      atomicAdd(&row[in ? (key[i] - lo) >> shift : (C > 1 ? 256u : 256u + (tid & 63))],
                in ? 1u : 0u);
    }
    __syncthreads();
    if constexpr (C > 1) {
      for (int b = tid; b < 256; b += NT) {
        uint32_t t = 0u;
#pragma unroll
        for (int c = 0; c < C; ++c) t += st.hist[c * kHistRow + b];
        st.total[b] = t;
      }
      __syncthreads();
    }
    if (tid < 64) find_bin(st, C > 1 ? st.total : st.hist);
    __syncthreads();
    lo = st.lo;
    hi = st.hi;
    whole = st.whole != 0u;
  }
  *lo_out = lo;
  *need_out = st.need;
  *whole_out = whole;
}

// Exact top-k search followed by the kept bitmap (in ks, after a barrier),
// with the units u < f_lo and u >= f_hi added to it; the caller emits the
// ranks it needs with emit_kept.
template <int KPT, int NW>
__device__ __forceinline__ void topk_bitmap(RadixState& st, KeptScratch<KPT, NW>& ks,
                                            const uint32_t (&key)[KPT], int U, int k,
                                            int f_lo = 0, int f_hi = 0x7FFFFFFF) {
  uint32_t T, need;
  bool whole;
  radix_search<KPT, NW>(st, key, U, k, &T, &need, &whole);
  kept_words<KPT, NW>(ks.mask, ks.tie, ks.base, key, U, T, need, whole, f_lo, f_hi, &ks.total);
}

}  // namespace sdkv
