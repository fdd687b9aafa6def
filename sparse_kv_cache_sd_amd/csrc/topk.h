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
// `need` keys equal to T in index order are kept.  Ballots and a scan in index
// order give every kept id its rank.  All counting is integer, so the result
// does not depend on thread timing.
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

// Bins 256 .. 319 are per-lane sinks: a key outside the interval adds 0 to
// its lane's sink instead of branching, so no single counter takes every
// lane's add (a divergent branch per key would serialise on gfx950).
constexpr int kHistWords = 256 + 64;

struct RadixState {
  uint32_t hist[kHistWords];
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
// key of [lo, hi], lanes covering bins from the top down, and narrow to it.
__device__ __forceinline__ void find_bin(RadixState& st) {
  const int lane = threadIdx.x & 63;
  const uint32_t need = st.need, lo = st.lo, hi = st.hi, shift = st.shift;
  uint32_t c[4], tot = 0u;
#pragma unroll
  for (int i = 0; i < 4; ++i) { c[i] = st.hist[255 - 4 * lane - i]; tot += c[i]; }
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

// Lanes below this one, as a 64-bit mask.
__device__ __forceinline__ uint64_t lanes_below() {
  return (1ull << (threadIdx.x & 63)) - 1ull;
}

// Rank of every kept unit among the kept units in ascending unit order, for
// keys held interleaved (key[i] of thread t is unit t + NT*i):
//   above(u) = key > T (key >= T for a whole bin), tie(u) = key == T otherwise,
//   A(u), Ties(u) = numbers of above / tie units with a smaller id,
//   kept(u) = above(u) or (tie(u) and Ties(u) < need),
//   rank(u) = A(u) + min(Ties(u), need).
// Per key slot i and wave w the above / tie counts go to LDS (s_cnt, 2 * KPT *
// NW words), one wave scans them in (i, w) order, and each wave ranks its
// lanes with ballots.  NW = 1 needs no barrier.
template <int KPT, int NW, typename Emit>
__device__ __forceinline__ void rank_kept(uint32_t* s_cnt, const uint32_t (&key)[KPT], int U,
                                          int k, uint32_t T, uint32_t need, bool whole,
                                          Emit&& emit) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int NT = NW * 64;
  const uint64_t below = lanes_below();
  if constexpr (NW == 1) {
    uint32_t a_run = 0u, t_run = 0u;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const bool v = lane + NT * i < U;
      const bool above = v && (whole ? key[i] >= T : key[i] > T);
      const bool tie = v && !whole && key[i] == T;
      const uint64_t ma = __ballot(above), mt = __ballot(tie);
      const uint32_t A = a_run + __popcll(ma & below);
      const uint32_t Ti = t_run + __popcll(mt & below);
      if (above || (tie && Ti < need)) {
        const uint32_t pos = A + min(Ti, need);
        if (pos < (uint32_t)k) emit((int)pos, lane + NT * i);
      }
      a_run += __popcll(ma);
      t_run += __popcll(mt);
    }
    return;
  } else {
    constexpr int PAIRS = KPT * NW;
    constexpr int PPL = (PAIRS + 63) / 64;  // (slot, wave) pairs per scanning lane
    static_assert(PPL <= 8, "at most 512 (slot, wave) pairs");
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const bool v = threadIdx.x + NT * i < U;
      const uint64_t ma = __ballot(v && (whole ? key[i] >= T : key[i] > T));
      const uint64_t mt = __ballot(v && !whole && key[i] == T);
      if (lane == 0) {
        s_cnt[2 * (i * NW + wave)] = __popcll(ma);
        s_cnt[2 * (i * NW + wave) + 1] = __popcll(mt);
      }
    }
    __syncthreads();
    if (wave == 0) {
      // lane holds pairs PPL lane .. PPL lane + PPL - 1 of the (slot, wave) order
      uint32_t ca[PPL], ct[PPL], sa = 0u, st = 0u;
#pragma unroll
      for (int q = 0; q < PPL; ++q) {
        const int e = PPL * lane + q;
        ca[q] = e < PAIRS ? s_cnt[2 * e] : 0u;
        ct[q] = e < PAIRS ? s_cnt[2 * e + 1] : 0u;
        sa += ca[q];
        st += ct[q];
      }
      uint32_t ea = wave_scan_dpp(sa) - sa, et = wave_scan_dpp(st) - st;
#pragma unroll
      for (int q = 0; q < PPL; ++q) {
        const int e = PPL * lane + q;
        if (e < PAIRS) { s_cnt[2 * e] = ea; s_cnt[2 * e + 1] = et; }
        ea += ca[q];
        et += ct[q];
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int u = threadIdx.x + NT * i;
      const bool v = u < U;
      const bool above = v && (whole ? key[i] >= T : key[i] > T);
      const bool tie = v && !whole && key[i] == T;
      const uint64_t ma = __ballot(above), mt = __ballot(tie);
      const uint32_t A = s_cnt[2 * (i * NW + wave)] + __popcll(ma & below);
      const uint32_t Ti = s_cnt[2 * (i * NW + wave) + 1] + __popcll(mt & below);
      if (above || (tie && Ti < need)) {
        const uint32_t pos = A + min(Ti, need);
        if (pos < (uint32_t)k) emit((int)pos, u);
      }
    }
  }
}

// Top-k by a whole block over keys held in registers, interleaved: key[i] of
// thread t is unit t + NT*i (keys past U are ignored).  emit(rank, unit) is
// called once per kept unit, rank = its position among the kept units in
// ascending unit order.
template <int KPT, int NW, typename Emit>
__device__ __forceinline__ void topk_regs(RadixState& st, uint32_t* s_cnt,
                                          const uint32_t (&key)[KPT], int U, int k, Emit&& emit) {
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
    if (tid < 256) st.hist[tid] = 0u;
    if (tid == 0) st.shift = shift;
    __syncthreads();
    // every thread adds 0 or 1 for every slot: no divergent branches
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const bool in = tid + NT * i < U && key[i] >= lo && key[i] <= hi;
      atomicAdd(&st.hist[in ? (key[i] - lo) >> shift : 256u + (tid & 63)], in ? 1u : 0u);
    }
    __syncthreads();
    if (tid < 64) find_bin(st);
    __syncthreads();
    lo = st.lo;
    hi = st.hi;
    whole = st.whole != 0u;
  }
  rank_kept<KPT, NW>(s_cnt, key, U, k, lo, st.need, whole, emit);
}

}  // namespace sdkv
