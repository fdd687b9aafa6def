// Stage 1b for many units (token unit at long context): exact top-k of the
// unit scores of one (sequence, KV head) spread over NB blocks, each owning a
// slice of kMSlice units.  The result is the same as the one-block selection
// (topk.h): the k largest scores, equal scores to the lower unit id, ids in
// ascending order ("SparDA ..." summary, Section 3.1 and Appendix A: the
// selected set).
//
// Three launches, every block of one (sequence, KV head) working on its slice:
//   hist: 2048 bins uniform in the score's value over [min, max] of the
//     scores (from the per-block partial minima and maxima); each block
//     writes the histogram of its slice.  Scores crowd a few exponents, so
//     bins of the value leave far fewer keys beside the k-th largest than
//     bins of the key's bits: about 200 of 131072 at 128K tokens, r 0.3, on
//     the synthetic inputs, where 11 key bits leave thousands.
//   collect: each block sums the slices' histograms, finds the bin b* that
//     holds the k-th largest score, and writes the number of its slice's keys
//     above b* and its keys in b* (key and unit: the candidates).
//   place: each block loads every candidate of its (sequence, KV head) and
//     ranks them (key descending, then unit ascending: equal scores go to the
//     lower id).  That gives the last kept candidate (T, t) and the kept
//     units of the slices before this one; the block keeps its units with
//     key > T, or key == T and unit <= t, and writes them in ascending order.
//     (In the token decode step the attention kernel runs this placement in
//     its own prologue instead: launch_select_multi_bins runs the first two.)
// The bin of a score is an fp32 subtract and multiply by the same constants
// in every block, then a clamp: monotone in the score, so every key above b*
// is above every candidate.  Where bins cannot be formed (k = 0 or U, all
// scores equal, a range that is not finite) or the candidates do not fit
// (kCapS per slice, kCapT per (sequence, KV head)), the place kernel finds
// the k-th largest key itself: MSD radix passes of 11 bits over every key of
// its (sequence, KV head), re-read from memory at each pass by every block of
// the group, then one pass that counts the kept units before its slice.
// Nothing here uses atomics outside LDS (counts only), so the result does not
// depend on timing.  Block ids are bg + B*Hkv*slice in every kernel here
// (device.h, group_block): all blocks of one (sequence, KV head) share an XCD,
// so the histograms and candidates they exchange stay in its L2.
#include "msel.h"

static_assert(sdkv::msel::kMSlice == sdkv::kSliceUnits, "one slice size");

namespace sdkv {

namespace {

using namespace msel;

__global__ __launch_bounds__(kMT) void msel_minmax_kernel(MArgs a, uint32_t* mm) {
  __shared__ uint32_t s_w[2][kMNW];
  const GroupBlock gbk = group_block(a.d.B * a.d.Hkv);
  const int blk = gbk.j, b = gbk.bg / a.d.Hkv;
  const int64_t bg = gbk.bg;
  const int s0 = blk * kMSlice;
  const float* sc = a.scores + bg * a.U_max;
  const int n = clamp_len(a.seq_lens[b], a.d.max_seq);
  const int U = min(a.unit == kPage ? (n + a.d.P - 1) / a.d.P : n, a.U_max);
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
  for (int i = 0; i < kMK; ++i) {
    const int u = s0 + (int)threadIdx.x + kMT * i;
    const uint32_t key = order_key(sc[min(u, a.U_max - 1)]);
    if (u < U) { mn = min(mn, key); mx = max(mx, key); }
  }
  mn = wave_umin(mn);
  mx = wave_umax(mx);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) { s_w[0][wave] = mn; s_w[1][wave] = mx; }
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int w = 1; w < kMNW; ++w) { mn = min(mn, s_w[0][w]); mx = max(mx, s_w[1][w]); }
    mm[(bg * a.NB + blk) * 2] = mn;
    mm[(bg * a.NB + blk) * 2 + 1] = mx;
  }
}

// Value histogram of each slice.
__global__ __launch_bounds__(kMT) void msel_hist_kernel(MArgs a) {
  __shared__ MShared sm;
  uint32_t key[kMK];
  const GroupBlock gbk = group_block(a.d.B * a.d.Hkv);
  const Group g = group_setup(a, sm, key, gbk.bg, gbk.j);
  if (!g.binned || g.s0 >= g.U) return;  // uniform per block
  for (int i = threadIdx.x; i < kMBins + 64; i += kMT) sm.hist[i] = 0u;
  __syncthreads();
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < kMK; ++i) {
    const bool v = g.s0 + (int)threadIdx.x + kMT * i < g.U;
    atomicAdd(&sm.hist[v ? vbin(g, key[i]) : (uint32_t)(kMBins + lane)], v ? 1u : 0u);
  }
  __syncthreads();
  // 16-bit counts (a slice holds kMSlice keys), four bins per thread in one
  // 8-byte store: half the bytes every collect block reads back
  static_assert(kMBins == 4 * kMT && kMSlice < 65536, "four 16-bit bins per thread");
  const int t4 = 4 * threadIdx.x;
  const uint2 packed = make_uint2(sm.hist[t4] | (sm.hist[t4 + 1] << 16),
                                  sm.hist[t4 + 2] | (sm.hist[t4 + 3] << 16));
  *reinterpret_cast<uint2*>(a.hist + (g.bg * a.NB + g.blk) * kMBins + t4) = packed;
}

// The bin b* of the k-th largest score; this slice's keys above it and in it.
__global__ __launch_bounds__(kMT) void msel_collect_kernel(MArgs a) {
  __shared__ MShared sm;
  uint32_t key[kMK];
  const GroupBlock gbk = group_block(a.d.B * a.d.Hkv);
  const Group g = group_setup(a, sm, key, gbk.bg, gbk.j);
  if (!g.binned || g.s0 >= g.U) return;  // uniform per block
  // sum the slices' histograms, kBPT bins per thread (one 8-byte load of
  // four 16-bit counts per slice), eight slices' loads issued together
  const int tid = threadIdx.x;
  const uint16_t* h = a.hist + g.bg * a.NB * kMBins;
  uint32_t c[kBPT] = {};
  for (int s0 = 0; s0 < g.nsl; s0 += 8) {
    uint2 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int s = min(s0 + i, g.nsl - 1);
      v[i] = *reinterpret_cast<const uint2*>(h + (int64_t)s * kMBins + (kMBins - kBPT - kBPT * tid));
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t m = s0 + i < g.nsl ? 0xFFFFu : 0u;
      // bins kMBins - 1 - kBPT tid - j, j = 0 .. 3: the last count first
      c[0] += (v[i].y >> 16) & m;
      c[1] += v[i].y & m;
      c[2] += (v[i].x >> 16) & m;
      c[3] += v[i].x & m;
    }
  }
  pick_bin(sm, c, (uint32_t)g.k);
  const uint32_t bstar = sm.sv[0];
  // this slice: keys above b*, and its keys in b* in (i, wave, lane) order
  const int lane = tid & 63, wave = tid >> 6;
  const uint64_t below = (1ull << lane) - 1ull;
  uint32_t above = 0u, inbin = 0u;
  uint32_t vb[kMK];
#pragma unroll
  for (int i = 0; i < kMK; ++i) {
    const bool v = g.s0 + tid + kMT * i < g.U;
    vb[i] = v ? vbin(g, key[i]) : 0u;
    above += (v && vb[i] > bstar) ? 1u : 0u;
    const bool in = v && vb[i] == bstar;
    inbin += in ? 1u : 0u;
    const uint64_t m = __ballot(in);
    if (lane == 0) sm.hist[i * kMNW + wave] = (uint32_t)__popcll(m);
  }
  __syncthreads();
  // offsets of the (i, wave) groups: one wave scans the kMK * kMNW counts
  if (wave == 0) {
    const uint32_t x = lane < kMK * kMNW ? sm.hist[lane] : 0u;
    const uint32_t inc = wave_scan_dpp(x);
    if (lane < kMK * kMNW) sm.hist[64 + lane] = inc - x;
  }
  __syncthreads();
  uint2* dst = a.cand + (g.bg * a.NB + g.blk) * kCapS;
#pragma unroll
  for (int i = 0; i < kMK; ++i) {
    const bool in = g.s0 + tid + kMT * i < g.U && vb[i] == bstar;
    const uint64_t m = __ballot(in);
    const uint32_t pos = sm.hist[64 + i * kMNW + wave] + (uint32_t)__popcll(m & below);
    if (in && pos < (uint32_t)kCapS) dst[pos] = make_uint2(key[i], (uint32_t)(g.s0 + tid + kMT * i));
  }
  block_sum2(sm, above, inbin);
  if (tid == 0) {
    a.above[g.bg * a.NB + g.blk] = above;
    a.ccount[g.bg * a.NB + g.blk] = inbin;
  }
}

// Kept ids of each slice at their place in the ascending list.
__global__ __launch_bounds__(kMT) void msel_place_kernel(MArgs a) {
  __shared__ MShared sm;
  __shared__ KeptScratch<kMK, kMNW> ks;
  // the counts and candidates are read with the group's setup
  const GroupBlock gbk = group_block(a.d.B * a.d.Hkv);
  const PlaceLoads pl = place_loads(a, gbk.bg);
  uint32_t key[kMK];
  const Group g = group_setup(a, sm, key, gbk.bg, gbk.j);
  const int tid = threadIdx.x;
  int32_t* out = a.sel_idx + g.bg * a.k_max;
  if (g.blk == 0 && tid == 0) a.sel_count[g.bg] = g.k;
  if (g.k == 0 || g.s0 >= g.U) return;  // uniform per block
  if (g.k == g.U) {
    for (int i = tid; i < kMSlice && g.s0 + i < g.U; i += kMT) out[g.s0 + i] = g.s0 + i;
    return;
  }
  uint32_t T, quota, base;
  bool whole;
  place_bounds(a, sm, g, pl, &T, &quota, &whole, &base);
  const int n_slice = min(kMSlice, g.U - g.s0);
  kept_words<kMK, kMNW>(ks.mask, ks.tie, ks.base, key, n_slice, T, quota, whole);
  emit_kept<kMK, kMNW>(ks.mask, ks.base, 0u, (uint32_t)kMSlice, [&](int pos, int u) {
    const uint32_t gp = base + (uint32_t)pos;
    if (gp < (uint32_t)g.k) out[gp] = g.s0 + u;
  });
}

}  // namespace

size_t msel_workspace_bytes(int B, int Hkv, int U_max) {
  const int64_t bg = (int64_t)B * Hkv;
  const int64_t NB = (U_max + kMSlice - 1) / kMSlice;
  return sizeof(uint32_t) * 2 * bg * NB + sizeof(uint16_t) * bg * NB * kMBins +
         sizeof(uint32_t) * 2 * bg * NB + sizeof(uint2) * bg * NB * kCapS;
}

namespace {

// The kernels' arguments and grid; mm_own: where the partial min / max keys
// go when they are computed here.
MArgs make_args(const SelectArgs& sa, void* ws, const int32_t* k_of, uint32_t** mm_own) {
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
  *mm_own = reinterpret_cast<uint32_t*>(p);
  p += sizeof(uint32_t) * 2 * bg * a.NB;
  a.hist = reinterpret_cast<uint16_t*>(p);
  p += sizeof(uint16_t) * bg * a.NB * kMBins;
  a.above = reinterpret_cast<uint32_t*>(p);
  p += sizeof(uint32_t) * bg * a.NB;
  a.ccount = reinterpret_cast<uint32_t*>(p);
  p += sizeof(uint32_t) * bg * a.NB;
  a.cand = reinterpret_cast<uint2*>(p);
  a.sel_idx = sa.sel_idx;
  a.sel_count = sa.sel_count;
  a.k_of = k_of;
  return a;
}

}  // namespace

hipError_t launch_select_multi(const SelectArgs& sa, const uint32_t* mm, int mm_nb, int mm_per,
                               void* ws, hipStream_t stream, const int32_t* k_of) {
  uint32_t* mm_own;
  MArgs a = make_args(sa, ws, k_of, &mm_own);
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
  msel_hist_kernel<<<grid, kMT, 0, stream>>>(a);
  msel_collect_kernel<<<grid, kMT, 0, stream>>>(a);
  msel_place_kernel<<<grid, kMT, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_select_multi_bins(const SelectArgs& sa, const uint32_t* mm, int mm_nb,
                                    int mm_per, void* ws, hipStream_t stream, SliceSel* out) {
  if (!mm || !out) return hipErrorInvalidValue;
  uint32_t* mm_own;
  MArgs a = make_args(sa, ws, nullptr, &mm_own);
  a.mm = mm;
  a.mm_nb = mm_nb;
  a.mm_per = mm_per;
  const dim3 grid(a.NB * sa.d.Hkv * sa.d.B);
  msel_hist_kernel<<<grid, kMT, 0, stream>>>(a);
  msel_collect_kernel<<<grid, kMT, 0, stream>>>(a);
  out->NB = a.NB;
  out->scores = a.scores;
  out->mm = a.mm;
  out->mm_nb = a.mm_nb;
  out->mm_per = a.mm_per;
  out->above = a.above;
  out->ccount = a.ccount;
  out->cand = a.cand;
  return hipGetLastError();
}

}  // namespace sdkv
