// Stage 1b for many units (token unit at long context): exact top-k of the
// unit scores of one (sequence, KV head) spread over NB blocks, each owning a
// slice of kMSlice units.  The result is the same as the one-block selection
// (topk.h): the k largest scores, equal scores to the lower unit id, ids in
// ascending order ("SparDA ..." summary, Section 3.1 and Appendix A: the
// selected set).
//
// An MSD radix select on the order-preserving 32-bit keys:
//   the key interval starts at [min, max] of the scores (per-block partial
//   minima and maxima, written by the token scorer or by a small kernel);
//   pass p (p = 0, 1, 2): every block first derives the interval [lo, hi] and
//     the count `need` still to take from it (from its own copy of the
//     previous pass's state and the per-block histograms, each block
//     redundantly), records that state in its own copy, and writes the
//     2048-bin histogram of its slice's keys inside [lo, hi] (bins of 2^shift
//     keys) and its number of keys above hi;
//   place: from the last histogram, the final state (a single key T, or a
//     bin kept whole) and, summed over the slices before this block, the keys
//     above T and equal to T; equal keys go to the lower id, so each block
//     knows its quota of them and where its ids go, and writes them in
//     ascending order.
// Three passes of 11 bits cover any 32-bit interval; a pass whose interval is
// settled returns at once.  Histograms are per block (no atomics), so the
// result does not depend on timing.  Block ids are bg + B*Hkv*slice in every
// kernel here (device.h, group_block): all blocks of one (sequence, KV head)
// share an XCD, so the histograms and states they exchange stay in its L2.
#include "topk.h"

namespace sdkv {

namespace {

constexpr int kMT = 512;               // threads per block
constexpr int kMNW = kMT / 64;
constexpr int kMK = 8;                 // keys per thread
constexpr int kMSlice = kMT * kMK;     // units per block
constexpr int kMBins = 2048;           // 11-bit bins
constexpr int kMPasses = 3;

struct MState {
  uint32_t lo, hi, need, whole, done, k, pad0, pad1;
};

struct MArgs {
  Dims d;
  int unit;
  const int32_t* seq_lens;
  const float* scores;       // [B][Hkv][U_max]
  int U_max, k_max, R_ppm, NB;
  const uint32_t* mm;        // [B*Hkv][mm_nb][2] partial min / max keys
  int mm_nb, mm_per;         // partials per (b, g); units per partial
  MState* st;                // [kMPasses][B*Hkv][NB] state at the start of each pass,
                             // one copy per block (read back by the same block id)
  uint32_t* over;            // [kMPasses][B*Hkv][NB] keys above hi per slice
  uint32_t* hist;            // [kMPasses][B*Hkv][NB][kMBins]
  int32_t* sel_idx;          // [B][Hkv][k_max]
  int32_t* sel_count;        // [B][Hkv]
  const int32_t* k_of;       // [B*Hkv] counts to keep, or NULL: min(keep_count(U), k_max)
};

struct MShared {
  RadixState rs;             // wa / wb: block scan scratch
  uint32_t hist[kMBins + 64];
  MState S;
  uint32_t red[4 * kMNW];
};

__device__ __forceinline__ int units_of(const MArgs& a, int b) {
  const int n = clamp_len(a.seq_lens[b], a.d.max_seq);
  return min(a.unit == kPage ? (n + a.d.P - 1) / a.d.P : n, a.U_max);
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

__device__ __forceinline__ uint32_t shift_of(uint32_t lo, uint32_t hi) {
  const uint32_t span = hi - lo;
  const int bits = span == 0u ? 0 : 32 - __clz(span);
  return bits > 11 ? bits - 11 : 0;
}

// Block sum of two counters (result in every thread).
__device__ __forceinline__ void block_sum2(MShared& sm, uint32_t& x, uint32_t& y) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  x = wave_sum(x);
  y = wave_sum(y);
  if (lane == 0) { sm.red[2 * wave] = x; sm.red[2 * wave + 1] = y; }
  __syncthreads();
  x = y = 0u;
#pragma unroll
  for (int w = 0; w < kMNW; ++w) { x += sm.red[2 * w]; y += sm.red[2 * w + 1]; }
  __syncthreads();
}

// State at the start of pass 0: [min, max] of the keys, need = k.
__device__ void initial_state(const MArgs& a, MShared& sm, int64_t bg, int U) {
  const int parts = min(a.mm_nb, (U + a.mm_per - 1) / a.mm_per);
  const uint32_t* mm = a.mm + bg * a.mm_nb * 2;
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
  for (int i = threadIdx.x; i < parts; i += kMT) {
    mn = min(mn, mm[2 * i]);
    mx = max(mx, mm[2 * i + 1]);
  }
  block_minmax<kMNW>(sm.rs, mn, mx);
  if (threadIdx.x == 0) {
    const int k = a.k_of ? min(max(a.k_of[bg], 0), U) : min(keep_count_dev(U, a.R_ppm), a.k_max);
    MState S{};
    S.lo = sm.rs.lo;
    S.hi = sm.rs.hi;
    S.need = (uint32_t)k;
    S.k = (uint32_t)k;
    S.whole = 0u;
    S.done = (k == 0 || k == U || S.lo >= S.hi) ? 1u : 0u;
    sm.S = S;
  }
  __syncthreads();
}

// Narrows `prev` with the histograms of pass p (summed over the NB slices):
// the bin holding the need-th largest key becomes the interval.  With
// blk >= 0 it also sums, over the slices before blk, the keys above the new
// interval and inside it (*above_before, *inside_before; every thread).
__device__ void narrow(const MArgs& a, MShared& sm, int64_t bg, int p, const MState prev,
                       int blk, uint32_t* above_before, uint32_t* inside_before) {
  const int tid = threadIdx.x;
  const uint32_t* h = a.hist + ((int64_t)p * a.d.B * a.d.Hkv + bg) * a.NB * kMBins;
  // thread t holds bins kMBins - 1 - BPT t - j (j < BPT): descending order;
  // its BPT bins are one vector load per slice
  constexpr int BPT = kMBins / kMT;
  static_assert(BPT == 2 || BPT == 4 || BPT == 8, "2, 4 or 8 bins per thread");
  typedef unsigned int vec_t __attribute__((ext_vector_type(BPT)));
  uint32_t c[BPT] = {}, cb[BPT] = {};
  for (int b0 = 0; b0 < a.NB; b0 += 8) {
    vec_t v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int s = min(b0 + i, a.NB - 1);
      v[i] = *reinterpret_cast<const vec_t*>(h + (int64_t)s * kMBins + (kMBins - BPT - BPT * tid));
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bool valid = b0 + i < a.NB, before = b0 + i < blk;
#pragma unroll
      for (int j = 0; j < BPT; ++j) {  // bin kMBins - 1 - BPT t - j is element BPT - 1 - j
        c[j] += valid ? v[i][BPT - 1 - j] : 0u;
        cb[j] += before ? v[i][BPT - 1 - j] : 0u;
      }
    }
  }
  uint32_t tot = 0u;
#pragma unroll
  for (int j = 0; j < BPT; ++j) tot += c[j];
  uint32_t run, unused;
  block_excl_scan2(sm.rs, tot, 0u, &run, &unused);  // keys in higher bins
  const uint32_t shift = shift_of(prev.lo, prev.hi);
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    if (run < prev.need && run + c[j] >= prev.need) {
      const uint32_t bin = (uint32_t)(kMBins - 1 - BPT * tid - j);
      MState S = prev;
      S.lo = prev.lo + (bin << shift);
      const uint64_t top = (uint64_t)S.lo + ((1ull << shift) - 1ull);
      S.hi = (uint32_t)(top < (uint64_t)prev.hi ? top : (uint64_t)prev.hi);
      S.need = prev.need - run;
      S.whole = c[j] == S.need ? 1u : 0u;
      S.done = (S.whole || S.lo == S.hi) ? 1u : 0u;
      sm.S = S;
      sm.red[4 * kMNW - 1] = (uint32_t)(BPT * tid + j);  // rank of the bin from the top
    }
    run += c[j];
  }
  __syncthreads();
  if (blk < 0) return;
  // slices before blk: keys in bins above the chosen one, and in it
  const uint32_t r = sm.red[4 * kMNW - 1];
  uint32_t ab = 0u, in = 0u;
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    const uint32_t rank = (uint32_t)(BPT * tid + j);
    ab += rank < r ? cb[j] : 0u;
    in += rank == r ? cb[j] : 0u;
  }
  __syncthreads();  // red[] is reused below
  block_sum2(sm, ab, in);
  *above_before = ab;
  *inside_before = in;
}

__global__ __launch_bounds__(kMT) void msel_minmax_kernel(MArgs a, uint32_t* mm) {
  __shared__ MShared sm;
  const GroupBlock gbk = group_block(a.d.B * a.d.Hkv);
  const int blk = gbk.j, b = gbk.bg / a.d.Hkv;
  const int64_t bg = gbk.bg;
  const int s0 = blk * kMSlice;
  uint32_t key[kMK];
  load_slice(a, bg, s0, key);
  const int U = units_of(a, b);
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
  for (int i = 0; i < kMK; ++i)
    if (s0 + (int)threadIdx.x + kMT * i < U) { mn = min(mn, key[i]); mx = max(mx, key[i]); }
  block_minmax<kMNW>(sm.rs, mn, mx);
  if (threadIdx.x == 0) {
    mm[(bg * a.NB + blk) * 2] = sm.rs.lo;
    mm[(bg * a.NB + blk) * 2 + 1] = sm.rs.hi;
  }
}

__global__ __launch_bounds__(kMT) void msel_pass_kernel(MArgs a, int p) {
  __shared__ MShared sm;
  const GroupBlock gbk = group_block(a.d.B * a.d.Hkv);
  const int blk = gbk.j, b = gbk.bg / a.d.Hkv;
  const int64_t bg = gbk.bg;
  const int64_t BG = (int64_t)a.d.B * a.d.Hkv;
  const int s0 = blk * kMSlice;
  uint32_t key[kMK];
  load_slice(a, bg, s0, key);
  const int U = units_of(a, b);
  if (p == 0) {
    initial_state(a, sm, bg, U);
  } else {
    const MState prev = a.st[((p - 1) * BG + bg) * a.NB + blk];
    if (prev.done) {
      if (threadIdx.x == 0) sm.S = prev;
      __syncthreads();
    } else {
      narrow(a, sm, bg, p - 1, prev, -1, nullptr, nullptr);
    }
  }
  const MState S = sm.S;
  if (threadIdx.x == 0) a.st[(p * BG + bg) * a.NB + blk] = S;
  if (S.done) return;
  const uint32_t shift = shift_of(S.lo, S.hi);
  for (int i = threadIdx.x; i < kMBins; i += kMT) sm.hist[i] = 0u;
  __syncthreads();
  const int lane = threadIdx.x & 63;
  uint32_t above = 0u;
#pragma unroll
  for (int i = 0; i < kMK; ++i) {
    const bool v = s0 + (int)threadIdx.x + kMT * i < U;
    const bool in = v && key[i] >= S.lo && key[i] <= S.hi;
    above += (v && key[i] > S.hi) ? 1u : 0u;
    atomicAdd(&sm.hist[in ? (key[i] - S.lo) >> shift : kMBins + lane], in ? 1u : 0u);
  }
  uint32_t unused = 0u;
  block_sum2(sm, above, unused);  // includes a barrier: the histogram is complete
  uint32_t* h = a.hist + ((p * BG + bg) * a.NB + blk) * kMBins;
  for (int i = threadIdx.x; i < kMBins; i += kMT) h[i] = sm.hist[i];
  if (threadIdx.x == 0) a.over[(p * BG + bg) * a.NB + blk] = above;
}

// Kept ids of each slice at their place in the ascending list.
__global__ __launch_bounds__(kMT) void msel_place_kernel(MArgs a) {
  __shared__ MShared sm;
  __shared__ KeptScratch<kMK, kMNW> ks;
  const GroupBlock gbk = group_block(a.d.B * a.d.Hkv);
  const int blk = gbk.j, b = gbk.bg / a.d.Hkv;
  const int64_t bg = gbk.bg;
  const int64_t BG = (int64_t)a.d.B * a.d.Hkv;
  const int s0 = blk * kMSlice;
  const int tid = threadIdx.x;
  uint32_t key[kMK];
  load_slice(a, bg, s0, key);
  const int U = units_of(a, b);
  // the last pass that built histograms
  int L = -1;
  MState prev = a.st[bg * a.NB + blk];
  for (int p = 0; p < kMPasses; ++p) {
    const MState s = a.st[(p * BG + bg) * a.NB + blk];
    if (!s.done) { L = p; prev = s; }
  }
  int32_t* out = a.sel_idx + bg * a.k_max;
  const uint32_t k = prev.k;
  if (blk == 0 && tid == 0) a.sel_count[bg] = (int32_t)k;
  if (k == 0u || s0 >= U) return;
  if ((int)k == U) {
    for (int i = tid; i < kMSlice && s0 + i < U; i += kMT) out[s0 + i] = s0 + i;
    return;
  }
  uint32_t above_before, equal_before;
  MState S;
  if (L < 0) {
    // every key equals lo: all are ties, the first k by id are kept
    S = prev;
    S.whole = 0u;
    above_before = 0u;
    equal_before = (uint32_t)s0;
  } else {
    // keys above hi_L in the slices before this one (loaded before the
    // narrowing so that the two reads overlap)
    uint32_t ov = 0u;
    for (int j = tid; j < blk; j += kMT) ov += a.over[(L * BG + bg) * a.NB + j];
    uint32_t ab, inb;
    narrow(a, sm, bg, L, prev, blk, &ab, &inb);
    S = sm.S;
    uint32_t unused = 0u;
    block_sum2(sm, ov, unused);
    above_before = ov + ab + (S.whole ? inb : 0u);
    equal_before = S.whole ? 0u : inb;
  }
  // max(need - equal_before, 0), as a signed difference (see kept_words)
  const uint32_t quota = (uint32_t)max((int)S.need - (int)equal_before, 0);
  const uint32_t base = above_before + min(equal_before, S.need);
  const int n_slice = min(kMSlice, U - s0);
  kept_words<kMK, kMNW>(ks.mask, ks.tie, ks.base, key, n_slice, S.lo, quota, S.whole != 0u);
  emit_kept<kMK, kMNW>(ks.mask, ks.base, 0u, (uint32_t)kMSlice, [&](int pos, int u) {
    const uint32_t gp = base + (uint32_t)pos;
    if (gp < k) out[gp] = s0 + u;
  });
}

}  // namespace

size_t msel_workspace_bytes(int B, int Hkv, int U_max) {
  const int64_t bg = (int64_t)B * Hkv;
  const int64_t NB = (U_max + kMSlice - 1) / kMSlice;
  return sizeof(uint32_t) * 2 * bg * NB + sizeof(MState) * kMPasses * bg * NB +
         sizeof(uint32_t) * kMPasses * bg * NB + sizeof(uint32_t) * kMPasses * bg * NB * kMBins;
}

hipError_t launch_select_multi(const SelectArgs& sa, const uint32_t* mm, int mm_nb, int mm_per,
                               void* ws, hipStream_t stream, const int32_t* k_of) {
  MArgs a{};
  a.d = sa.d;
  a.unit = sa.unit;
  a.seq_lens = sa.seq_lens;
  a.scores = sa.unit_scores;
  a.U_max = sa.U_max;
  a.k_max = sa.k_max;
  a.R_ppm = sa.R_ppm;
  a.NB = (sa.U_max + kMSlice - 1) / kMSlice;
  const int64_t bg = (int64_t)sa.d.B * sa.d.Hkv;
  char* p = static_cast<char*>(ws);
  uint32_t* mm_own = reinterpret_cast<uint32_t*>(p);
  p += sizeof(uint32_t) * 2 * bg * a.NB;
  a.st = reinterpret_cast<MState*>(p);
  p += sizeof(MState) * kMPasses * bg * a.NB;
  a.over = reinterpret_cast<uint32_t*>(p);
  p += sizeof(uint32_t) * kMPasses * bg * a.NB;
  a.hist = reinterpret_cast<uint32_t*>(p);
  a.sel_idx = sa.sel_idx;
  a.sel_count = sa.sel_count;
  a.k_of = k_of;
  const dim3 grid(a.NB * sa.d.Hkv * sa.d.B);  // block id = bg + B*Hkv*slice
  if (mm) {
    a.mm = mm;
    a.mm_nb = mm_nb;
    a.mm_per = mm_per;
  } else {
    msel_minmax_kernel<<<grid, kMT, 0, stream>>>(a, mm_own);
    a.mm = mm_own;
    a.mm_nb = a.NB;
    a.mm_per = kMSlice;
  }
  for (int pass = 0; pass < kMPasses; ++pass) msel_pass_kernel<<<grid, kMT, 0, stream>>>(a, pass);
  msel_place_kernel<<<grid, kMT, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace sdkv
