// The steps of the many-block exact top-k (units beyond one block's
// registers) that more than one kernel runs: select_multi.hip runs them as
// three launches (hist, collect, place), and in token unit the attention
// kernel can run the placement in its own prologue.  See select_multi.hip
// for the method.
#pragma once

#include <cfloat>

#include "topk.h"

namespace sdkv {
namespace msel {
namespace {

constexpr int kMT = 512;               // threads per block
constexpr int kMNW = kMT / 64;
constexpr int kMK = 8;                 // keys per thread
constexpr int kMSlice = kMT * kMK;     // units per block
constexpr int kMBins = 2048;           // value bins (collect, place); 11-bit bins (fallback)
constexpr int kBPT = kMBins / kMT;     // bins per thread when a block scans them
constexpr int kCapS = 64;              // candidates a slice hands on
constexpr int kCapT = 1024;            // candidates of one (sequence, KV head)
constexpr int kMaxSlices = 512;        // slices per (sequence, KV head) the binned path takes
constexpr int kCR = 8;                 // candidate slots per thread read with the setup
static_assert(kBPT == 4, "a thread scans four bins");

struct MArgs {
  Dims d;
  int unit;
  const int32_t* seq_lens;
  const float* scores;       // [B][Hkv][U_max]
  int U_max, k_max, R_ppm, NB;
  const uint32_t* mm;        // [B*Hkv][mm_nb][2] partial min / max keys
  int mm_nb, mm_per;         // partials per (b, g); units per partial
  uint16_t* hist;            // [B*Hkv][NB][kMBins] value histogram of each slice (<= 4096 a bin)
  uint32_t* above;           // [B*Hkv][NB] keys above bin b* in each slice
  uint32_t* ccount;          // [B*Hkv][NB] keys in bin b* in each slice
  uint2* cand;               // [B*Hkv][NB][kCapS] (key, unit) of the first of them
  int32_t* sel_idx;          // [B][Hkv][k_max]
  int32_t* sel_count;        // [B][Hkv]
  const int32_t* k_of;       // [B*Hkv] counts to keep, or NULL: min(keep_count(U), k_max)
};

struct MShared {
  uint32_t hist[kMBins + 64];  // + a sink word per lane for keys outside the range
  uint32_t wa[kMNW], wb[kMNW], wc[kMNW], wd[kMNW];
  uint32_t cnt[kMaxSlices], off[kMaxSlices + 1];
  // candidates as key << 32 | ~unit: a larger value ranks first (larger key,
  // then lower unit); zero past the last (never ranks above one)
  uint64_t comp[kCapT + 8];
  uint32_t rank[kCapT];
  uint32_t sv[8];
};

// inverse of order_key (+0 for the key of -0)
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// The (sequence, KV head) of this block and what every block of it derives
// alike: its count to keep, the key range of its scores and the value bins.
struct Group {
  int64_t bg;
  int blk, s0, U, k, nsl;
  uint32_t kmin, kmax;
  float vmin, inv;  // bin of value v: min((v - vmin) * inv, 2047)
  bool binned;
};

__device__ __forceinline__ uint32_t vbin(const Group& g, uint32_t key) {
  const float t = (key_value(key) - g.vmin) * g.inv;
  return t >= (float)(kMBins - 1) ? (uint32_t)(kMBins - 1) : (uint32_t)t;
}

// Block sums of two counters (every thread gets them).
__device__ __forceinline__ void block_sum2(MShared& sm, uint32_t& x, uint32_t& y) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  x = wave_sum(x);
  y = wave_sum(y);
  __syncthreads();  // wa / wb may still be read from a previous call
  if (lane == 0) { sm.wa[wave] = x; sm.wb[wave] = y; }
  __syncthreads();
  x = y = 0u;
#pragma unroll
  for (int w = 0; w < kMNW; ++w) { x += sm.wa[w]; y += sm.wb[w]; }
}

// Exclusive block scan of one counter, in thread order; *total gets the sum.
__device__ __forceinline__ uint32_t block_excl_scan(MShared& sm, uint32_t v, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t inc = wave_scan_dpp(v);
  __syncthreads();
  if (lane == 63) sm.wa[wave] = inc;
  __syncthreads();
  uint32_t before = 0u, all = 0u;
#pragma unroll
  for (int w = 0; w < kMNW; ++w) {
    before += w < wave ? sm.wa[w] : 0u;
    all += sm.wa[w];
  }
  *total = all;
  return before + inc - v;
}

// Keys of this block's slice, interleaved (key[i] of thread t is slice unit
// t + kMT * i), loaded unconditionally.
__device__ __forceinline__ void load_slice(const MArgs& a, int64_t bg, int s0,
                                           uint32_t (&key)[kMK]) {
  const float* sc = a.scores + bg * a.U_max;
#pragma unroll
  for (int i = 0; i < kMK; ++i)
    key[i] = order_key(sc[min(s0 + (int)threadIdx.x + kMT * i, a.U_max - 1)]);
}

// Partial minima and maxima a thread reads in the first round (more in a
// loop after it).
constexpr int kMMR = 4;

// Every block starts with the same round of loads, none waiting for another:
// the sequence length, the group's partial minima and maxima (all of them,
// masked once the length is known) and the keys of slice blk of group bg.
__device__ Group group_setup(const MArgs& a, MShared& sm, uint32_t (&key)[kMK], int64_t bg,
                             int blk) {
  Group g;
  g.bg = bg;
  g.blk = blk;
  g.s0 = g.blk * kMSlice;
  const int b = (int)(bg / a.d.Hkv);
  const int tid = threadIdx.x;
  const int n_raw = a.seq_lens[b];
  const uint32_t* mm = a.mm + g.bg * a.mm_nb * 2;
  uint2 part[kMMR];
#pragma unroll
  for (int r = 0; r < kMMR; ++r)
    part[r] = *reinterpret_cast<const uint2*>(mm + 2 * min(tid + kMT * r, a.mm_nb - 1));
  load_slice(a, g.bg, g.s0, key);
  const int n = clamp_len(n_raw, a.d.max_seq);
  g.U = min(a.unit == kPage ? (n + a.d.P - 1) / a.d.P : n, a.U_max);
  g.k = a.k_of ? min(max(a.k_of[g.bg], 0), g.U) : min(keep_count_dev(g.U, a.R_ppm), a.k_max);
  g.nsl = (g.U + kMSlice - 1) / kMSlice;
  const int parts = min(a.mm_nb, (g.U + a.mm_per - 1) / a.mm_per);
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
  for (int r = 0; r < kMMR; ++r) {
    if (tid + kMT * r < parts) {
      mn = min(mn, part[r].x);
      mx = max(mx, part[r].y);
    }
  }
  for (int i = tid + kMT * kMMR; i < parts; i += kMT) {
    mn = min(mn, mm[2 * i]);
    mx = max(mx, mm[2 * i + 1]);
  }
  mn = wave_umin(mn);
  mx = wave_umax(mx);
  const int lane = tid & 63, wave = tid >> 6;
  if (lane == 0) { sm.wa[wave] = mn; sm.wb[wave] = mx; }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kMNW; ++w) { mn = min(mn, sm.wa[w]); mx = max(mx, sm.wb[w]); }
  g.kmin = mn;
  g.kmax = mx;
  g.vmin = key_value(mn);
  const float w = key_value(mx) - g.vmin;
  g.inv = (float)kMBins / w;
  // w and inv finite and positive (false for NaN as well)
  g.binned = g.k > 0 && g.k < g.U && mn < mx && w > 0.f && w <= FLT_MAX && g.inv > 0.f &&
             g.inv <= FLT_MAX && g.nsl <= kMaxSlices;
  return g;
}

__device__ __forceinline__ uint32_t shift_of(uint32_t lo, uint32_t hi) {
  const uint32_t span = hi - lo;
  const int bits = span == 0u ? 0 : 32 - __clz(span);
  return bits > 11 ? bits - 11 : 0;
}

// The bin holding the need-th largest of the keys counted in c (thread t
// holds bins kMBins - 1 - kBPT t - j, j < kBPT: descending order).  Sets
// sm.sv[0] = bin, sm.sv[1] = keys in higher bins, sm.sv[2] = keys in it;
// every thread reads them after the barrier.
__device__ __forceinline__ void pick_bin(MShared& sm, const uint32_t (&c)[kBPT], uint32_t need) {
  uint32_t tot = 0u;
#pragma unroll
  for (int j = 0; j < kBPT; ++j) tot += c[j];
  uint32_t all;
  uint32_t run = block_excl_scan(sm, tot, &all);  // keys in higher bins
#pragma unroll
  for (int j = 0; j < kBPT; ++j) {
    if (run < need && run + c[j] >= need) {
      sm.sv[0] = (uint32_t)(kMBins - 1 - kBPT * (int)threadIdx.x - j);
      sm.sv[1] = run;
      sm.sv[2] = c[j];
    }
    run += c[j];
  }
  __syncthreads();
}

// Without usable bins or candidates: the k-th largest key T of the group by
// MSD radix passes over every key (re-read from memory), then the kept units
// before this slice.  kept = key > T, plus the first `quota` keys equal to T
// of this slice in unit order; whole: kept = key >= T.
__device__ void select_all(const MArgs& a, MShared& sm, const Group& g, uint32_t* T,
                           uint32_t* quota, bool* whole, uint32_t* base) {
  const int tid = threadIdx.x, lane = tid & 63;
  const float* sc = a.scores + g.bg * a.U_max;
  uint32_t lo = g.kmin, hi = g.kmax, need = (uint32_t)g.k;
  bool wh = false;
  // 11 bits per pass: 32 -> 21 -> 10 -> 0 bits of span in at most three
  for (int p = 0; p < 3 && lo < hi && !wh; ++p) {  // uniform
    const uint32_t shift = shift_of(lo, hi);
    __syncthreads();  // the previous pass's readers are done with hist
    for (int i = tid; i < kMBins + 64; i += kMT) sm.hist[i] = 0u;
    __syncthreads();
    for (int u0 = 0; u0 < g.U; u0 += kMT * 8) {
      uint32_t kk[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) kk[r] = order_key(sc[min(u0 + tid + kMT * r, g.U - 1)]);
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const bool in = u0 + tid + kMT * r < g.U && kk[r] >= lo && kk[r] <= hi;
        atomicAdd(&sm.hist[in ? (kk[r] - lo) >> shift : (uint32_t)(kMBins + lane)], in ? 1u : 0u);
      }
    }
    __syncthreads();
    uint32_t c[kBPT];
#pragma unroll
    for (int j = 0; j < kBPT; ++j) c[j] = sm.hist[kMBins - 1 - kBPT * tid - j];
    pick_bin(sm, c, need);
    const uint32_t bin = sm.sv[0], run = sm.sv[1], cnt = sm.sv[2];
    const uint32_t nlo = lo + (bin << shift);
    const uint64_t top = (uint64_t)nlo + ((1ull << shift) - 1ull);
    hi = (uint32_t)(top < (uint64_t)hi ? top : (uint64_t)hi);
    lo = nlo;
    need -= run;
    wh = cnt == need;
  }
  // kept units before this slice
  uint32_t ab = 0u, eq = 0u;
  for (int u0 = 0; u0 < g.s0; u0 += kMT * 8) {
    uint32_t kk[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) kk[r] = order_key(sc[min(u0 + tid + kMT * r, g.s0 - 1)]);
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const bool v = u0 + tid + kMT * r < g.s0;
      ab += (v && (wh ? kk[r] >= lo : kk[r] > lo)) ? 1u : 0u;
      eq += (v && !wh && kk[r] == lo) ? 1u : 0u;
    }
  }
  block_sum2(sm, ab, eq);
  *T = lo;
  *whole = wh;
  *quota = wh ? 0u : (uint32_t)max((int)need - (int)eq, 0);
  *base = ab + (wh ? 0u : min(eq, need));
}

// What placement reads for group bg before anything is known: thread t's
// slice's counts (slice t) and the group's first kCR * kMT candidate slots
// (masked later; slots past them are read after the counts).
struct PlaceLoads {
  uint32_t as_raw, cs_raw;
  uint2 cv[kCR];
  const uint2* src;
};

__device__ __forceinline__ PlaceLoads place_loads(const MArgs& a, int64_t bg) {
  PlaceLoads pl;
  const int tid = threadIdx.x;
  const int tsl = min(tid, a.NB - 1);
  pl.as_raw = a.above[bg * a.NB + tsl];
  pl.cs_raw = a.ccount[bg * a.NB + tsl];
  pl.src = a.cand + bg * a.NB * kCapS;
  const int nslots = a.NB * kCapS;
#pragma unroll
  for (int r = 0; r < kCR; ++r) pl.cv[r] = pl.src[min(tid + kMT * r, nslots - 1)];
  return pl;
}

// The kept set as seen from slice g.blk, for 0 < k < U: every key above T is
// kept, and of the keys equal to T the first *quota of the slice in unit
// order (*whole: every key >= T, quota 0); *base is the number of kept units
// in the slices before it.  From the candidates of the bin b* when they fit,
// else by radix passes over every key of the group (select_all).
__device__ void place_bounds(const MArgs& a, MShared& sm, const Group& g, const PlaceLoads& pl,
                             uint32_t* T_out, uint32_t* quota_out, bool* whole_out,
                             uint32_t* base_out) {
  const int tid = threadIdx.x;
  bool fallback = !g.binned;
  uint32_t T = 0u, quota = 0u, base = 0u;
  bool whole = false;
  if (g.binned) {
    // every slice's counts (thread s reads slice s: nsl <= kMT): keys above
    // b* before this slice and in all, slices over kCapS, and the offsets of
    // the candidates in the gathered list -- one barrier pair for all four
    static_assert(kMaxSlices <= kMT, "a thread per slice");
    const int lane = tid & 63, wave = tid >> 6;
    const bool mine = tid < g.nsl;
    const uint32_t as = mine ? pl.as_raw : 0u, cs = mine ? pl.cs_raw : 0u;
    const uint32_t cc = min(cs, (uint32_t)kCapS);
    uint32_t ab = wave_sum(tid < g.blk ? as : 0u), atot = wave_sum(as);
    const uint32_t over = wave_sum(cs > (uint32_t)kCapS ? 1u : 0u);
    const uint32_t inc = wave_scan_dpp(cc);
    __syncthreads();  // the setup's readers of wa / wb are done
    if (lane == 63) { sm.wa[wave] = ab; sm.wb[wave] = atot; sm.wc[wave] = over; sm.wd[wave] = inc; }
    __syncthreads();
    ab = atot = 0u;
    uint32_t ov = 0u, off = inc - cc, ctot = 0u;
#pragma unroll
    for (int w = 0; w < kMNW; ++w) {
      ab += sm.wa[w];
      atot += sm.wb[w];
      ov += sm.wc[w];
      off += w < wave ? sm.wd[w] : 0u;
      ctot += sm.wd[w];
    }
    fallback = ov != 0u || ctot > (uint32_t)kCapT;
    if (!fallback) {
      if (mine) {
        sm.cnt[tid] = cc;
        sm.off[tid] = off;
      }
      const int nc = (int)ctot, nc8 = (nc + 7) & ~7;
      if (tid < nc8 - nc) sm.comp[nc + tid] = 0ull;
      for (int c = tid; c < nc; c += kMT) sm.rank[c] = 0u;
      __syncthreads();
      // gather the candidates: slot x = (slice x / kCapS, entry x % kCapS)
      const int used = g.nsl * kCapS;
      auto comp_of = [](uint2 v) { return ((uint64_t)v.x << 32) | (uint64_t)(~v.y); };
#pragma unroll
      for (int r = 0; r < kCR; ++r) {
        const int x = tid + kMT * r, sl = x / kCapS, e = x - sl * kCapS;
        if (x < used && (uint32_t)e < sm.cnt[sl]) sm.comp[sm.off[sl] + e] = comp_of(pl.cv[r]);
      }
      for (int x = tid + kMT * kCR; x < used; x += kMT) {
        const int sl = x / kCapS, e = x - sl * kCapS;
        if ((uint32_t)e < sm.cnt[sl]) sm.comp[sm.off[sl] + e] = comp_of(pl.src[x]);
      }
      __syncthreads();
      // rank of each candidate = the candidates above it.  With fewer
      // candidates than threads, P threads share one candidate's comparisons
      // (an interval of the others each, eight read at a time) and add their
      // counts in LDS.
      const int P = nc >= kMT ? 1 : kMT / max(nc, 1);
      const int span = ((nc8 + P - 1) / P + 7) & ~7;
      for (int t = tid; t < nc * P; t += kMT) {
        const int c = t % nc, part = t / nc;
        const uint64_t me = sm.comp[c];
        const int o1 = min((part + 1) * span, nc8);
        uint32_t r = 0u;
        for (int o = part * span; o < o1; o += 8) {
          uint64_t x[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) x[j] = sm.comp[o + j];
#pragma unroll
          for (int j = 0; j < 8; ++j) r += x[j] > me ? 1u : 0u;
        }
        atomicAdd(&sm.rank[c], r);
      }
      __syncthreads();
      const uint32_t need = (uint32_t)g.k - atot;  // >= 1: b* holds the k-th largest
      uint32_t kb = 0u;  // kept candidates of the slices before this one
      for (int c = tid; c < nc; c += kMT) {
        const uint32_t r = sm.rank[c];
        const uint64_t me = sm.comp[c];
        const uint32_t unit = ~(uint32_t)me;
        if (r + 1u == need) { sm.sv[4] = (uint32_t)(me >> 32); sm.sv[5] = unit; }
        kb += (r < need && (int)unit < g.s0) ? 1u : 0u;
      }
      __syncthreads();
      T = sm.sv[4];
      const uint32_t t_unit = sm.sv[5];
      // ties of this slice that are kept: equal to T with unit <= t
      uint32_t q = 0u;
      for (int c = tid; c < nc; c += kMT) {
        const uint64_t x = sm.comp[c];
        const uint32_t unit = ~(uint32_t)x;
        q += ((uint32_t)(x >> 32) == T && (int)unit >= g.s0 && (int)unit < g.s0 + kMSlice &&
              unit <= t_unit)
                 ? 1u
                 : 0u;
      }
      block_sum2(sm, kb, q);
      quota = q;
      base = ab + kb;
    }
  }
  if (fallback) {
    select_all(a, sm, g, T_out, quota_out, whole_out, base_out);
    return;
  }
  *T_out = T;
  *quota_out = quota;
  *whole_out = whole;
  *base_out = base;
}

}  // namespace
}  // namespace msel
}  // namespace sdkv
