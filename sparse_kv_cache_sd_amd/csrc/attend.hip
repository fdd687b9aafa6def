// Stage 2: split-K attention over the kept units, and the log-sum-exp merge
// of the splits.
//
// Dense and sparse decoding share these kernels ("Where Activation Sparsity
// and KV-Cache Sparsity Cross in LLM Decoding", list view, Abstract): a dense
// call is the same kernel with every unit kept.  Attention runs over the
// tokens of the kept blocks only ("SparDA ..." summary, Section 3.1).
//
// Work split: block (j, g, b) owns kept-list entries [j*E, (j+1)*E) of the
// (sequence b, KV head g) list.  Its tokens are cut into chunks of 16 rows: a
// 16-token page is one chunk, a 64-token page four, and in token unit a chunk
// is 16 consecutive list entries.  Each split keeps an online softmax (running
// max m, sum l, weighted value sum) per query head of the group and writes
// its normalised output and log-sum-exp; a second kernel merges the splits of
// every head by log-sum-exp.  (A merge inside the last block to finish would
// need an agent-scope release per block, which on gfx950 writes back the
// XCD's L2 each time and costs more than the kernel boundary.)
//
// The kept list comes from memory (a selection computed before), is the
// identity (dense), or is computed by the block itself from the page scores:
// every split of (b, g) runs the same exact top-k (topk.h, all eight waves)
// and keeps its slice, which saves a kernel launch and a round trip through
// memory.  In token unit past one block's selection the block instead places
// the kept units of its range of one slice from the many-block top-k's
// candidates (msel.h), the last step of that top-k.
//
// bf16 kernel (matrix cores).  Per chunk and wave:
//   S^T[t][h] = sum_c K[t][c] Q[h][c]   4 x mfma 16x16x32 bf16 (d = 128): K rows
//                                       are the A operand straight from HBM, the
//                                       group's queries (padded to 16 heads) the
//                                       B operand kept in registers;
//   p = exp2(S^T * scale * log2 e - m)  in the MFMA result layout (lane holds 4
//                                       tokens of one head); the chunk max over
//                                       16 tokens uses two gfx950 permlane swaps;
//   O^T[c][h] += sum_t V^T[c][t] P^T[t][h]   mfma 16x16x16 bf16 per 16 channels,
//                                       P split into bf16 hi + lo parts so the
//                                       weights keep ~16 significant bits; V^T
//                                       comes from V rows staged in LDS through
//                                       the gfx950 transposing LDS read.
// Row addresses of up to 16 chunks per wave are resolved first (list entry,
// then block table) into LDS, then K/V loads run two chunks at a time,
// double-buffered.  The fp32 kernel keeps the same split structure with
// vector FMAs.
#include "msel.h"

namespace sdkv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));


constexpr int kAttendWaves = 8;     // waves per block
// Chunks a wave resolves per round (list entry, then block table): 8 when a
// wave holds many chunks (fewer dependent rounds), 4 when it holds at most 4
// (the 13-page splits of a 32K-token sequence kept at 0.2 with 8 KV heads:
// 25.6 -> 24.9 us per step; 8 is better for long lists and dense, 75.9
// against 78.0 us at 1M tokens).  Softmax attention over 9 to 16 chunks per
// wave resolves them all at once, so no wave stalls on a second round for
// its last few chunks: the V gather at 128K tokens kept at 0.3 (10 chunks a
// wave) 27.5 -> 25.9 us, the 1M-token page attention (13) 58.0 -> 57.2 us.
constexpr int kResolveWide = 8, kResolveNarrow = 4, kResolveLong = 16;

// What a block does with the attended tokens' logits.
enum WeightMode : int {
  kWSoftmax = 0,  // online softmax (running max, exp2)
  kWEntmax = 1,   // alpha-entmax weights against a precomputed threshold
  kWLogits = 2    // no attention: write the logits out (V is not read)
};

// How a block obtains its kept list.
enum SelMode : int {
  kListed = 0,     // from memory (sel_idx) or the identity
  kSliced = 1,     // token unit: placed in the kernel from the many-block top-k's candidates
  kBlock4 = 4,     // in-kernel top-k by the whole block, 4 / 8 / 32 keys per thread
  kBlock8 = 8,
  kBlock32 = 32
};

// A block's slice of the list, known without device loads: entries
// [e0, e_hi) may be read (e_hi <= list length); chunks past the loaded
// count are masked later.
struct Span {
  int e0, e_hi;
  int nch;  // chunks the slice can hold
};

__device__ __forceinline__ Span span_of(const AttendArgs& a, int j, int list_len) {
  Span sp;
  sp.e0 = j * a.E;
  sp.e_hi = min(sp.e0 + a.E, list_len);
  const int ne = max(0, sp.e_hi - sp.e0);
  sp.nch = a.unit == kPage ? ne * (a.d.P / 16) : (ne + 15) / 16;
  return sp;
}

// Without a list: the identity (every unit), or with a window the last
// keep_count(U) units -- list entry e is unit window_start + e.
__device__ __forceinline__ int window_start(const AttendArgs& a, int U) {
  return a.window ? U - keep_count_dev(U, a.R_ppm) : 0;
}

// Pool rows (row-major [num_pages * H_kv * P] index) of row `row` of N
// chunks c[i] (or -1 where that row is not attended; tok[i] receives its
// token id).  unit_at(e) returns list entry e for e < sp.e_hi.  Every read is
// issued unconditionally with a clamped index, list entries first and block
// table entries second, so the N lookups cost two memory round trips.
template <int N, typename UnitAt>
__device__ __forceinline__ void resolve_rows(const AttendArgs& a, const Span& sp,
                                             UnitAt&& unit_at, int cnt, int n, int U, int b,
                                             int g, const int (&c)[N], const bool (&live)[N],
                                             int row, int (&pr)[N], int (&tok)[N]) {
  const Dims& d = a.d;
  const bool pg = a.unit == kPage;
  const int cpu = d.P / 16;
  int e[N], v[N], phys[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    e[i] = pg ? sp.e0 + c[i] / cpu : sp.e0 + c[i] * 16 + row;
    v[i] = unit_at(max(sp.e0, min(e[i], sp.e_hi - 1)));
  }
#pragma unroll
  for (int i = 0; i < N; ++i) {
    tok[i] = pg ? v[i] * d.P + (c[i] - (c[i] / cpu) * cpu) * 16 + row : v[i];
    int lp = tok[i] / d.P;
    lp = lp < 0 ? 0 : (lp >= d.max_pages ? d.max_pages - 1 : lp);
    phys[i] = a.block_table[(int64_t)b * d.max_pages + lp];
  }
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int lp = tok[i] / d.P;
    const bool ok = live[i] && e[i] < sp.e_hi && e[i] < cnt && v[i] >= 0 && (!pg || v[i] < U) &&
                    tok[i] < n && phys[i] >= 0 && phys[i] < d.num_pages;
    pr[i] = ok ? (int)(((int64_t)phys[i] * d.Hkv + g) * d.P + (tok[i] - lp * d.P)) : -1;
  }
}

// Writes a block's partial (s_po [G][D], s_plse [G] in LDS); split 0 of
// (0, 0) also records the split count for the merge kernel.
template <int D, int G, int NT>
__device__ __forceinline__ void write_partial(const AttendArgs& a, int b, int g, int j,
                                              const float* s_po, const float* s_plse) {
  const int tid = threadIdx.x;
  const int64_t bh0 = (int64_t)b * a.d.Hq + g * G;
  for (int i = tid * 4; i < G * D; i += NT * 4) {
    const int h = i / D, c = i - h * D;
    *reinterpret_cast<float4*>(&a.part_o[((bh0 + h) * a.S + j) * D + c]) =
        *reinterpret_cast<const float4*>(&s_po[i]);
  }
  if (tid < G) a.part_lse[(bh0 + tid) * a.S + j] = s_plse[tid];
  if (tid == 0 && j == 0 && g == 0 && b == 0) *a.split_count = a.S;
}

// Log-sum-exp merge of the S split partials of one (sequence, query head):
// M = max_j lse_j, w_j = exp(lse_j - M), out = sum_j w_j o_j / sum_j w_j,
// lse = M + log sum_j w_j; splits with lse = -inf weigh nothing.  One block
// of 256 threads per (sequence, query head): thread (slice, c4) sums float4
// column c4 over the splits j = slice (mod SLICES), issuing the loads of its
// first splits before the weights are known; the slices add up in LDS.
template <int D>
__global__ __launch_bounds__(256) void merge_splits_kernel(MergeArgs a) {
  constexpr int NT = 256, C4 = D / 4, SLICES = NT / C4, PRE = 8;
  __shared__ float s_w[kMaxSplits];
  __shared__ float s_ML[2];
  __shared__ float4 s_red[SLICES][C4];
  // block id = bg + B*Hkv*i merges head i of group bg: on the XCD that wrote
  // the group's partials
  const GroupBlock gb = group_block(a.d.B * a.d.Hkv);
  const int64_t bh = (int64_t)(gb.bg / a.d.Hkv) * a.d.Hq + (gb.bg % a.d.Hkv) * a.d.G + gb.j;
  const int tid = threadIdx.x, lane = tid & 63;
  const float* __restrict__ part_o = a.part_o;
  const float* __restrict__ part_lse = a.part_lse;
  float* __restrict__ out = a.out;
  float* __restrict__ lse = a.lse;
  const int S = a.S_known > 0 ? a.S_known : min(max(*a.split_count, 1), a.S_max);
  const float* pl = part_lse + bh * S;
  const int c4 = tid % C4, slice = tid / C4;
  const float4* po = reinterpret_cast<const float4*>(part_o + bh * S * D) + c4;
  float4 pre[PRE];
#pragma unroll
  for (int i = 0; i < PRE; ++i) {
    const int j = slice + i * SLICES;
    pre[i] = j < S ? po[(int64_t)j * C4] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  if (tid < 64) {
    float M = -INFINITY;
    for (int j = lane; j < S; j += 64) M = fmaxf(M, pl[j]);
    M = wave_max(M);
    float L = 0.f;
    for (int j = lane; j < S; j += 64) {
      const float w = M == -INFINITY ? 0.f : expf(pl[j] - M);
      s_w[j] = w;
      L += w;
    }
    L = wave_sum(L);
    if (lane == 0) { s_ML[0] = M; s_ML[1] = L; }
  }
  __syncthreads();
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int i = 0; i < PRE; ++i) {
    const int j = slice + i * SLICES;
    const float w = j < S ? s_w[j] : 0.f;
    acc.x = fmaf(w, pre[i].x, acc.x);
    acc.y = fmaf(w, pre[i].y, acc.y);
    acc.z = fmaf(w, pre[i].z, acc.z);
    acc.w = fmaf(w, pre[i].w, acc.w);
  }
#pragma unroll 4
  for (int j = slice + PRE * SLICES; j < S; j += SLICES) {
    const float w = s_w[j];
    const float4 v = po[(int64_t)j * C4];
    acc.x = fmaf(w, v.x, acc.x);
    acc.y = fmaf(w, v.y, acc.y);
    acc.z = fmaf(w, v.z, acc.z);
    acc.w = fmaf(w, v.w, acc.w);
  }
  s_red[slice][c4] = acc;
  __syncthreads();
  if (tid < C4) {
    float4 sum = s_red[0][tid];
#pragma unroll
    for (int s = 1; s < SLICES; ++s) {
      const float4 v = s_red[s][tid];
      sum.x += v.x; sum.y += v.y; sum.z += v.z; sum.w += v.w;
    }
    const float L = s_ML[1];
    const float inv = L > 0.f ? 1.f / L : 0.f;
    reinterpret_cast<float4*>(out + bh * D)[tid] =
        make_float4(sum.x * inv, sum.y * inv, sum.z * inv, sum.w * inv);
    if (tid == 0) lse[bh] = L > 0.f ? s_ML[0] + logf(L) : -INFINITY;
  }
}

// ----------------------------------------------------------------------------
// bf16: matrix-core kernel
// ----------------------------------------------------------------------------

template <int D, int G, bool LOGITS, int SEL, int WM, int RW>
__global__ __launch_bounds__(kAttendWaves * 64) void attend_mfma_kernel(AttendArgs a) {
  constexpr int NW = kAttendWaves, NT = NW * 64;
  static_assert(RW == 4 || RW == 8 || RW == 16, "resolve windows of 4, 8 or 16 chunks");
  constexpr int KS = D / 32;        // 16x16x32 steps over the channels
  constexpr int CT = D / 16;        // 16-channel output tiles
  constexpr int VROW = D + 8;       // staged V row, bf16 elements (16-byte aligned rows)
  constexpr bool SLICED = SEL == kSliced;
  constexpr bool SELECTS = SEL != kListed && !SLICED;  // page top-k in the kernel
  constexpr bool LOCAL = SELECTS || SLICED;            // the list is built in LDS
  constexpr int KEYS = SELECTS ? SEL : 1;
  constexpr int KK = SLICED ? msel::kMK : KEYS;        // keys per thread of the kept bitmap
  static_assert(!SLICED || (LOGITS && WM == kWSoftmax && NW == msel::kMNW),
                "placement: softmax over stored logits, one placement block");
  constexpr bool TOK = LOGITS || WM == kWLogits;  // rows' token ids are kept
  static_assert(WM != kWEntmax || LOGITS, "entmax weights read stored logits");
  static_assert(WM != kWLogits || !LOGITS, "logits are computed from K");
  // The V staging area is reused after the chunk loop for the per-wave outputs.
  constexpr int kStage = NW * 16 * VROW * 2;
  constexpr int kAfter = NW * G * D * 4;
  __shared__ __align__(16) unsigned char s_raw[kStage > kAfter ? kStage : kAfter];
  __shared__ int s_rows[NW][RW][16];
  __shared__ int s_tok[TOK ? NW : 1][RW][16];
  __shared__ float s_m[NW][16], s_l[NW][16];
  __shared__ __align__(16) float s_po[G * D];
  __shared__ float s_plse[G];
  __shared__ int s_list[SLICED ? kSliceUnits : (SELECTS ? kMaxSelectE : 1)];
  __shared__ RadixState s_rs;
  __shared__ msel::MShared s_ms;
  __shared__ KeptScratch<LOCAL ? KK : 1, NW> s_kept;
  auto s_v = reinterpret_cast<bf16_t(*)[16 * VROW]>(s_raw);
  auto s_o = reinterpret_cast<float(*)[G][D]>(s_raw);

  const Dims& d = a.d;
  const GroupBlock gb = group_block(d.B * d.Hkv);
  const int j = gb.j, g = gb.bg % d.Hkv, b = gb.bg / d.Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = lane & 15, quad = lane >> 4;
  const int64_t bg = (int64_t)b * d.Hkv + g;
  const bf16_t* kp = static_cast<const bf16_t*>(a.k_pages);
  const bf16_t* vp = static_cast<const bf16_t*>(a.v_pages);
  const int32_t* list = a.sel_idx ? a.sel_idx + bg * a.k_max : nullptr;
  const int units_cap = a.unit == kPage ? d.max_pages : d.max_seq;
  Span sp = span_of(a, j, (list || LOCAL || a.window) ? a.k_max : units_cap);

  // In-kernel selection: the scores of (b, g) are read before the sequence
  // length is known (a row holds max_pages of them).
  uint32_t key[KEYS];
  if constexpr (SELECTS) {
    // interleaved: key[i] of thread t is unit t + NT*i
    const float* sc = a.unit_scores + bg * d.max_pages;
#pragma unroll
    for (int i = 0; i < KEYS; ++i)
      key[i] = order_key(sc[min((int)threadIdx.x + NT * i, d.max_pages - 1)]);
  }
  const int n = clamp_len(a.seq_lens[b], d.max_seq);
  const int U = a.unit == kPage ? (n + d.P - 1) / d.P : n;
  int cnt;
  int w0 = 0;  // first unit of a window
  if constexpr (SELECTS) {
    const int k = min(keep_count_dev(U, a.R_ppm), a.k_max);
    int32_t* full = (j == 0 && a.sel_out) ? a.sel_out + bg * a.k_max : nullptr;
    auto emit = [&](int pos, int unit_id) {
      if (pos >= sp.e0 && pos < sp.e_hi) s_list[pos - sp.e0] = unit_id;
      if (full) full[pos] = unit_id;
    };
    // kept: the top-k, plus the first force_init and last force_local units
    const int f_lo = min(a.force_init, U), f_hi = max(U - a.force_local, 0);
    int kept = k;
    if (k == U) {
      for (int e = threadIdx.x; e < U; e += NT) emit(e, e);
    } else if (k > 0) {
      topk_bitmap<KEYS, NW>(s_rs, s_kept, key, U, k, f_lo, f_hi);
      kept = min((int)s_kept.total, a.k_max);
      // this split's slice of the ranks, or all of them when split 0 also
      // writes the selection out
      emit_kept<KEYS, NW>(s_kept.mask, s_kept.base, full ? 0u : (uint32_t)sp.e0,
                          full ? (uint32_t)kept : (uint32_t)sp.e_hi, emit);
    }
    if (j == 0 && a.sel_count_out && threadIdx.x == 0) a.sel_count_out[bg] = kept;
    cnt = kept;
    __syncthreads();
  } else if constexpr (SLICED) {
    // The placement of the many-block top-k for slice j >> sub_log2 (every
    // block of the slice alike), then the kept units of this split's range
    // into the LDS list, in unit order, and to sel_out at their place.
    msel::MArgs ma{};
    ma.d = d;
    ma.unit = a.unit;
    ma.seq_lens = a.seq_lens;
    ma.scores = a.sl.scores;
    ma.U_max = units_cap;
    ma.k_max = a.k_max;
    ma.R_ppm = a.R_ppm;
    ma.NB = a.sl.NB;
    ma.mm = a.sl.mm;
    ma.mm_nb = a.sl.mm_nb;
    ma.mm_per = a.sl.mm_per;
    ma.above = const_cast<uint32_t*>(a.sl.above);
    ma.ccount = const_cast<uint32_t*>(a.sl.ccount);
    ma.cand = const_cast<uint2*>(a.sl.cand);
    const int slice = j >> a.sub_log2, sub = j - (slice << a.sub_log2);
    const msel::PlaceLoads pl = msel::place_loads(ma, bg);
    uint32_t mkey[msel::kMK];
    const msel::Group gr = msel::group_setup(ma, s_ms, mkey, bg, slice);
    const int R = kSliceUnits >> a.sub_log2;  // units of this split
    constexpr int W = msel::kMK * NW;         // bitmap words of a slice
    const int wd0 = (sub * R) >> 6, wd1 = ((sub + 1) * R) >> 6;
    int32_t* full = a.sel_out ? a.sel_out + bg * a.k_max : nullptr;
    if (j == 0 && a.sel_count_out && threadIdx.x == 0) a.sel_count_out[bg] = gr.k;
    int kept = 0;
    if (gr.k > 0 && gr.s0 < gr.U) {  // uniform
      const int u_lo = gr.s0 + sub * R;
      if (gr.k == gr.U) {
        kept = max(0, min(R, gr.U - u_lo));
        for (int e = threadIdx.x; e < kept; e += NT) {
          s_list[e] = u_lo + e;
          if (full) full[u_lo + e] = u_lo + e;
        }
      } else {
        uint32_t T, quota, base;
        bool whole;
        msel::place_bounds(ma, s_ms, gr, pl, &T, &quota, &whole, &base);
        kept_words<msel::kMK, NW>(s_kept.mask, s_kept.tie, s_kept.base, mkey,
                                  min(kSliceUnits, gr.U - gr.s0), T, quota, whole, 0,
                                  0x7FFFFFFF, &s_kept.total);
        // ranks in the slice of the range's first and last kept units
        const uint32_t r_lo = wd0 < W ? s_kept.base[wd0] : s_kept.total;
        const uint32_t r_hi = wd1 < W ? s_kept.base[wd1] : s_kept.total;
        kept = (int)(r_hi - r_lo);
        emit_kept<msel::kMK, NW>(s_kept.mask, s_kept.base, r_lo, r_hi, [&](int pos, int u) {
          s_list[pos - (int)r_lo] = gr.s0 + u;
          const uint32_t gp = base + (uint32_t)pos;
          if (full && gp < (uint32_t)gr.k) full[gp] = gr.s0 + u;
        });
      }
    }
    cnt = kept;
    sp.e0 = 0;
    sp.e_hi = kept;
    sp.nch = (kept + 15) / 16;
    __syncthreads();
  } else {
    w0 = window_start(a, U);
    cnt = list ? min(a.sel_count[bg], a.k_max) : U - w0;
  }
  // chunks [w_lo, w_hi) of this block belong to this wave
  const int cpw = (sp.nch + NW - 1) / NW;
  const int w_lo = min(sp.nch, wave * cpw), w_hi = min(sp.nch, w_lo + cpw);
  auto unit_at = [&](int e) -> int {
    if constexpr (LOCAL) return e < cnt ? s_list[e - sp.e0] : -1;
    else {
      // one unconditional load (a valid dummy address in identity mode)
      const int v = *(list ? list + e : a.seq_lens + b);
      return list ? v : w0 + e;
    }
  };

  // B operand of the score product: lane holds Q[h = row][32 s + 8 quad .. +7].
  bf16x8_t qop[KS];
  {
    const bf16_t* qrow =
        static_cast<const bf16_t*>(a.q) + ((int64_t)b * d.Hq + g * G + min(row, G - 1)) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4_t w = *reinterpret_cast<const u32x4_t*>(qrow + 32 * s + 8 * quad);
      if (LOGITS || row >= G) w = u32x4_t{0u, 0u, 0u, 0u};
      qop[s] = __builtin_bit_cast(bf16x8_t, w);
    }
  }
  const float qs = d.scale * kLog2e;
  // a valid row-sized address for loads of rows that are not attended
  const bf16_t* qrow0 = static_cast<const bf16_t*>(a.q) + ((int64_t)b * d.Hq + g * G) * D;
  // stored logits of head `row` of the group (token unit): token t's is
  // logit_row[t * logit_st] (the public [B][Hq][max_seq] layout, or
  // token-major [B][Hkv][max_seq][G] inside a decode step)
  const float* logit_row =
      !LOGITS ? nullptr
      : a.logits_tm ? a.token_logits + ((int64_t)b * d.Hkv + g) * d.max_seq * G + min(row, G - 1)
                    : a.token_logits + ((int64_t)b * d.Hq + g * G + min(row, G - 1)) * d.max_seq;
  const int logit_st = a.logits_tm ? G : 1;
  // slot of the split's first row (slot-indexed logits): chunk c of the
  // split holds slots slot0 + 16 c .. + 15
  const int slot0 = sp.e0 * (a.unit == kPage ? d.P : 1);

  float4_t acc[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) acc[ct] = float4_t{0.f, 0.f, 0.f, 0.f};
  // Entmax weights are absolute (no running max): m stays 0 and l sums them.
  float m = WM == kWEntmax ? 0.f : -INFINITY, l = 0.f;
  const float tau_row =
      WM == kWEntmax ? a.tau[(int64_t)b * d.Hq + g * G + min(row, G - 1)] : 0.f;
  float* logit_out_row =
      WM == kWLogits ? a.logits_out + ((int64_t)b * d.Hq + g * G + min(row, G - 1)) * d.max_seq
                     : nullptr;
  bf16_t* sv = &s_v[wave][0];

  // One 16-row chunk: scores, weights, value accumulation.  lg holds the
  // chunk's stored logits (rows 4 quad + r of head `row`) when LOGITS; tk
  // holds those rows' token ids when logits are written out.
  auto process = [&](const u32x4_t (&kv)[KS], const u32x4_t (&vv)[KS], const float (&lg)[4],
                     const int (&tk)[4], uint32_t vmask, int ci) {
    if constexpr (WM != kWLogits) {
#pragma unroll
      for (int s = 0; s < KS; ++s)
        *reinterpret_cast<u32x4_t*>(sv + row * VROW + 32 * s + 8 * quad) = vv[s];
    }
    float4_t st = {0.f, 0.f, 0.f, 0.f};
    if constexpr (!LOGITS) {
#pragma unroll
      for (int s = 0; s < KS; ++s)
        st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kv[s]), qop[s],
                                                      st, 0, 0, 0);
    }
    if constexpr (WM == kWLogits) {
      if (row < G) {
        if (a.logits_slots) {
          // the chunk's 16 slots: attended rows get their logit, the rest -inf
#pragma unroll
          for (int r = 0; r < 4; ++r)
            logit_out_row[slot0 + ci * 16 + 4 * quad + r] =
                ((vmask >> (4 * quad + r)) & 1u) ? st[r] * d.scale : -INFINITY;
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if ((vmask >> (4 * quad + r)) & 1u) logit_out_row[tk[r]] = st[r] * d.scale;
        }
      }
      return;
    }
    float p[4];
    if constexpr (WM == kWEntmax) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        p[r] = row < G && ((vmask >> (4 * quad + r)) & 1u)
                   ? entmax_weight(fmaf(a.alpha_m1, lg[r], -tau_row), a.beta)
                   : 0.f;
      l += (p[0] + p[1]) + (p[2] + p[3]);
    } else {
      float x[4];
      if constexpr (!LOGITS) {
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] = st[r] * qs;
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] = row < G ? lg[r] * kLog2e : 0.f;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (!((vmask >> (4 * quad + r)) & 1u)) x[r] = -INFINITY;
      float cm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
      cm = max_xor32(cm);
      cm = max_xor16(cm);
      const float mn = fmaxf(m, cm);
      const float alpha = exp2f(m - mn);
#pragma unroll
      for (int r = 0; r < 4; ++r) p[r] = exp2f(x[r] - mn);
      l = fmaf(l, alpha, (p[0] + p[1]) + (p[2] + p[3]));
      if (alpha != 1.f) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) acc[ct] *= alpha;
      }
      m = mn;
    }
    short4_t phi, plo;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const __bf16 hi = (__bf16)p[r];
      const __bf16 lo = (__bf16)(p[r] - (float)hi);
      phi[r] = __builtin_bit_cast(short, hi);
      plo[r] = __builtin_bit_cast(short, lo);
    }
    __builtin_amdgcn_wave_barrier();
    // lane reads V[4 quad + row / 4][16 ct + 4 (row % 4) .. +3]; the transposing
    // read hands it V[4 quad + r][16 ct + row] for r = 0..3 (the V^T operand).
    const bf16_t* vsrc = sv + (4 * quad + (row >> 2)) * VROW + 4 * (row & 3);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const short4_t vop = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) short4_t*)(vsrc + 16 * ct));
      acc[ct] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vop, phi, acc[ct], 0, 0, 0);
      acc[ct] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vop, plo, acc[ct], 0, 0, 0);
    }
    __builtin_amdgcn_wave_barrier();
  };

  for (int r0 = w_lo; r0 < w_hi; r0 += RW) {
    const int nc = min(RW, w_hi - r0);
    // Resolve the rows of up to RW chunks: lane (row, quad) takes chunk it*4+quad.
    {
      constexpr int NR = RW / 4;
      int cc[NR], pr[NR], tk[NR];
      bool live[NR];
#pragma unroll
      for (int it = 0; it < NR; ++it) {
        cc[it] = r0 + it * 4 + quad;
        live[it] = it * 4 + quad < nc;
      }
      resolve_rows<NR>(a, sp, unit_at, cnt, n, U, b, g, cc, live, row, pr, tk);
#pragma unroll
      for (int it = 0; it < NR; ++it) {
        s_rows[wave][it * 4 + quad][row] = pr[it];
        if constexpr (TOK) s_tok[wave][it * 4 + quad][row] = tk[it];
      }
    }
    __builtin_amdgcn_wave_barrier();
    // Entmax weights are exactly zero below the threshold, and most kept
    // chunks hold no token above it: the window's logits are read first
    // (one round of loads), and a chunk whose every weight is zero is
    // skipped -- its V is not read, and it would add nothing.
    uint32_t live_chunks = 0xFFFFFFFFu;
    if constexpr (WM == kWEntmax) {
      float zl[RW][4];
      bool rv[RW][4];
#pragma unroll
      for (int c = 0; c < RW; ++c) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          int t = s_tok[wave][c][4 * quad + r];
          t = t < 0 ? 0 : (t >= d.max_seq ? d.max_seq - 1 : t);
          rv[c][r] = s_rows[wave][c][4 * quad + r] >= 0;
          zl[c][r] = a.logits_slots
                         ? logit_row[min(slot0 + (r0 + c) * 16 + 4 * quad + r, d.max_seq - 1)]
                         : logit_row[(int64_t)t * logit_st];
        }
      }
      live_chunks = 0u;
#pragma unroll
      for (int c = 0; c < RW; ++c) {
        bool any = false;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          any = any || (row < G && rv[c][r] && fmaf(a.alpha_m1, zl[c][r], -tau_row) > 0.f);
        live_chunks |= (__ballot(any) != 0ull ? 1u : 0u) << c;
      }
    }

    // Two chunks per load batch, double-buffered: batch i+1 is in flight while
    // batch i is processed.  Every load is issued unconditionally (rows that
    // are not attended read the group's query row, which is cached, and are
    // masked), so the compiler can wait for one batch while the next stays in
    // flight; a branch around a load would make it drain all of them.
    u32x4_t kA[2][KS], vA[2][KS], kB[2][KS], vB[2][KS];
    float lA[2][4], lB[2][4];
    int tA[2][4], tB[2][4];
    uint32_t mA[2], mB[2];
    auto load2 = [&](u32x4_t (&kk)[2][KS], u32x4_t (&vv)[2][KS], float (&ll)[2][4],
                     int (&tt)[2][4], uint32_t (&mm)[2], int c0) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int c = c0 + i;
        int pr = s_rows[wave][min(c, RW - 1)][row];
        if (c >= nc || !((live_chunks >> min(c, 31)) & 1u)) pr = -1;
        mm[i] = (uint32_t)(__ballot(pr >= 0) & 0xFFFFull);
        const bf16_t* kr = pr >= 0 ? kp + (int64_t)pr * D : qrow0;
        const bf16_t* vr = pr >= 0 ? vp + (int64_t)pr * D : qrow0;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          if constexpr (!LOGITS) kk[i][s] = *reinterpret_cast<const u32x4_t*>(kr + 32 * s + 8 * quad);
          else kk[i][s] = u32x4_t{0u, 0u, 0u, 0u};
          if constexpr (WM != kWLogits) vv[i][s] = *reinterpret_cast<const u32x4_t*>(vr + 32 * s + 8 * quad);
          else vv[i][s] = u32x4_t{0u, 0u, 0u, 0u};
        }
        if constexpr (TOK) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            int t = s_tok[TOK ? wave : 0][min(c, RW - 1)][4 * quad + r];
            t = t < 0 ? 0 : (t >= d.max_seq ? d.max_seq - 1 : t);
            tt[i][r] = t;
            if constexpr (LOGITS)
              ll[i][r] = a.logits_slots
                             ? logit_row[min(slot0 + (r0 + c) * 16 + 4 * quad + r, d.max_seq - 1)]
                             : logit_row[(int64_t)t * logit_st];
            else ll[i][r] = 0.f;
          }
        }
      }
    };
    // (slot-indexed logits only: the logits-only pass also visits the
    // window's chunks that attend nothing, to write their -inf slots)
    auto run2 = [&](u32x4_t (&kk)[2][KS], u32x4_t (&vv)[2][KS], float (&ll)[2][4],
                    int (&tt)[2][4], uint32_t (&mm)[2], int c0) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
        if (mm[i] != 0u || (WM == kWLogits && a.logits_slots && c0 + i < nc))
          process(kk[i], vv[i], ll[i], tt[i], mm[i], r0 + c0 + i);
    };
    load2(kA, vA, lA, tA, mA, 0);
    for (int c = 0;; c += 4) {
      load2(kB, vB, lB, tB, mB, c + 2);
      run2(kA, vA, lA, tA, mA, c);
      if (c + 2 >= nc) break;
      load2(kA, vA, lA, tA, mA, c + 4);
      run2(kB, vB, lB, tB, mB, c + 2);
      if (c + 4 >= nc) break;
    }
  }
  if constexpr (WM == kWLogits) return;

  // lane (row, quad) holds head `row`: sum over the four quads of l; the
  // running max is already shared by them.
  l = sum_xor32(l);
  l = sum_xor16(l);
  __syncthreads();  // every wave is done with the staging area
  if (quad == 0) { s_m[wave][row] = m; s_l[wave][row] = l; }
  if (row < G) {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int r = 0; r < 4; ++r) s_o[wave][row][16 * ct + 4 * quad + r] = acc[ct][r];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < G * D; i += NT) {
    const int h = i / D, c = i - h * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, s_m[w][h]);
    float L = 0.f, A = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float f = s_m[w][h] == -INFINITY ? 0.f : exp2f(s_m[w][h] - M);
        L = fmaf(s_l[w][h], f, L);
        A = fmaf(s_o[w][h][c], f, A);
      }
    }
    s_po[i] = L > 0.f ? A / L : 0.f;
    if (c == 0) s_plse[h] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
  }
  __syncthreads();
  write_partial<D, G, NT>(a, b, g, j, s_po, s_plse);
}

// ----------------------------------------------------------------------------
// fp32: vector kernel (same split structure; list from memory or identity)
// ----------------------------------------------------------------------------

template <int D, int G>
__global__ __launch_bounds__(kAttendWaves * 64) void attend_f32_kernel(AttendArgs a) {
  constexpr int NW = kAttendWaves, NT = NW * 64;
  constexpr int LPR = D / 8;   // lanes per row, 8 channels each
  constexpr int RPW = 64 / LPR;
  __shared__ float s_m[NW][RPW][G], s_l[NW][RPW][G];
  __shared__ __align__(16) float s_acc[NW][G][D];
  __shared__ __align__(16) float s_po[G * D];
  __shared__ float s_plse[G];

  const Dims& d = a.d;
  const GroupBlock gb = group_block(d.B * d.Hkv);
  const int j = gb.j, g = gb.bg % d.Hkv, b = gb.bg / d.Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane / LPR, cl = lane % LPR;
  const int64_t bg = (int64_t)b * d.Hkv + g;
  const float* kp = static_cast<const float*>(a.k_pages);
  const float* vp = static_cast<const float*>(a.v_pages);
  const bool use_logits = a.token_logits != nullptr;
  const bool ent = a.tau != nullptr;          // entmax weights (with use_logits)
  const bool wl = a.logits_out != nullptr;    // write logits, no attention
  const int32_t* list = a.sel_idx ? a.sel_idx + bg * a.k_max : nullptr;
  const int units_cap = a.unit == kPage ? d.max_pages : d.max_seq;
  const Span sp = span_of(a, j, (list || a.window) ? a.k_max : units_cap);
  const int n = clamp_len(a.seq_lens[b], d.max_seq);
  const int U = a.unit == kPage ? (n + d.P - 1) / d.P : n;
  const int w0 = list ? 0 : window_start(a, U);
  const int cnt = list ? min(a.sel_count[bg], a.k_max) : U - w0;
  auto unit_at = [&](int e) -> int {
    const int v = *(list ? list + e : a.seq_lens + b);
    return list ? v : w0 + e;
  };

  // scores in the exp2 domain, or natural logits when they are written out
  const float qs = wl ? d.scale : d.scale * kLog2e;
  float qv[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    load8(static_cast<const float*>(a.q) + ((int64_t)b * d.Hq + g * G + h) * D + cl * 8, qv[h]);
#pragma unroll
    for (int c = 0; c < 8; ++c) qv[h][c] *= qs;
  }
  float tauv[G];
#pragma unroll
  for (int h = 0; h < G; ++h) tauv[h] = ent ? a.tau[(int64_t)b * d.Hq + g * G + h] : 0.f;
  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = ent ? 0.f : -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[h][c] = 0.f;
  }
  const int rows = sp.nch * 16;
  for (int base = wave * RPW; base < rows; base += NW * RPW) {
    const int r = base + sub;
    int cc[1] = {r >> 4}, prr[1], tk[1];
    const bool live[1] = {r < rows};
    resolve_rows<1>(a, sp, unit_at, cnt, n, U, b, g, cc, live, r & 15, prr, tk);
    const int pr = prr[0], t = tk[0];
    const bool ok = pr >= 0;
    const int64_t off = (int64_t)pr * D + cl * 8;
    float s[G];
    if (use_logits) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const int64_t at = a.logits_tm ? (((int64_t)b * d.Hkv + g) * d.max_seq + t) * G + h
                                       : ((int64_t)b * d.Hq + g * G + h) * d.max_seq + t;
        const float z = ok ? a.token_logits[at] : 0.f;
        s[h] = ent ? z : z * kLog2e;
      }
    } else {
      float kv[8];
      if (ok) {
        load8(kp + off, kv);
      } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) kv[c] = 0.f;
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float dot = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) dot = fmaf(qv[h][c], kv[c], dot);
        s[h] = group_sum<LPR>(dot);
      }
    }
    if (wl) {
      if (ok) {
        float mine = 0.f;
#pragma unroll
        for (int h = 0; h < G; ++h)
          if (h == cl) mine = s[h];
        if (cl < G) a.logits_out[((int64_t)b * d.Hq + g * G + cl) * d.max_seq + t] = mine;
      }
      continue;
    }
    if (ok && ent) {
      float vv[8];
      load8(vp + off, vv);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float p = entmax_weight(fmaf(a.alpha_m1, s[h], -tauv[h]), a.beta);
        l[h] += p;
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[h][c] = fmaf(p, vv[c], acc[h][c]);
      }
    } else if (ok) {
      float vv[8];
      load8(vp + off, vv);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float mn = fmaxf(m[h], s[h]);
        const float alpha = exp2f(m[h] - mn);
        const float p = exp2f(s[h] - mn);
        l[h] = fmaf(l[h], alpha, p);
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[h][c] = fmaf(acc[h][c], alpha, p * vv[c]);
        m[h] = mn;
      }
    }
  }
  if (wl) return;
  // per wave: lane-rows to LDS, merged below together with the other waves
  if (cl == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) { s_m[wave][sub][h] = m[h]; s_l[wave][sub][h] = l[h]; }
  }
  __syncthreads();
  float M[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    M[h] = -INFINITY;
    for (int w = 0; w < NW; ++w)
      for (int q = 0; q < RPW; ++q) M[h] = fmaxf(M[h], s_m[w][q][h]);
  }
  // each lane-row rescales to the block max, then rows of a wave add up in LDS
  for (int h = 0; h < G; ++h) {
    const float f = m[h] == -INFINITY ? 0.f : exp2f(m[h] - M[h]);
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[h][c] *= f;
  }
  for (int q = 0; q < RPW; ++q) {
    if (sub == q) {
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          float* dst = &s_acc[wave][h][cl * 8 + c];
          *dst = (q == 0 ? 0.f : *dst) + acc[h][c];
        }
    }
    __syncthreads();
  }
  for (int i = threadIdx.x; i < G * D; i += NT) {
    const int h = i / D, c = i - h * D;
    float L = 0.f, A = 0.f;
    if (M[h] != -INFINITY) {
      for (int w = 0; w < NW; ++w) {
        A += s_acc[w][h][c];
        for (int q = 0; q < RPW; ++q)
          L += s_m[w][q][h] == -INFINITY ? 0.f : s_l[w][q][h] * exp2f(s_m[w][q][h] - M[h]);
      }
    }
    s_po[i] = L > 0.f ? A / L : 0.f;
    if (c == 0) s_plse[h] = L > 0.f ? (M[h] + log2f(L)) * kLn2 : -INFINITY;
  }
  __syncthreads();
  write_partial<D, G, NT>(a, b, g, j, s_po, s_plse);
}

// Keys per thread the in-kernel selection uses for max_pages units: the whole
// block selects (a single wave's dependent instruction chain is slower).
static int select_mode(int max_pages) {
  if (max_pages <= kAttendWaves * 64 * 4) return kBlock4;
  if (max_pages <= kAttendWaves * 64 * 8) return kBlock8;
  return kBlock32;
}

// One launch of the matrix-core kernel with the resolve window for the
// split's chunks per wave (cpw).
template <int D, int G, bool LOGITS, int SEL, int WM>
static void go_mfma(const AttendArgs& a, dim3 grid, hipStream_t st, int64_t cpw) {
  constexpr int NT = kAttendWaves * 64;
  if (cpw <= kResolveNarrow) {
    attend_mfma_kernel<D, G, LOGITS, SEL, WM, kResolveNarrow><<<grid, NT, 0, st>>>(a);
    return;
  }
  if constexpr (WM == kWSoftmax) {
    if (cpw > kResolveWide && cpw <= kResolveLong) {
      attend_mfma_kernel<D, G, LOGITS, SEL, WM, kResolveLong><<<grid, NT, 0, st>>>(a);
      return;
    }
  }
  attend_mfma_kernel<D, G, LOGITS, SEL, WM, kResolveWide><<<grid, NT, 0, st>>>(a);
}

hipError_t launch_attend(const AttendArgs& a, hipStream_t st) {
  const Dims& d = a.d;
  if (a.S < 1 || a.S > kMaxSplits) return hipErrorInvalidValue;
  const bool selects = a.unit_scores != nullptr;
  if (a.window && (selects || a.sel_idx)) return hipErrorInvalidValue;
  if ((a.force_init | a.force_local) < 0) return hipErrorInvalidValue;
  if (selects && (a.unit != kPage || a.sel_idx != nullptr || d.dtype != kBF16 ||
                  a.E > kMaxSelectE || d.max_pages > kMaxSelectU))
    return hipErrorInvalidValue;
  const dim3 grid(a.S * d.Hkv * d.B);  // block id = bg + B*Hkv*j (XCD-aware)
  const bool logits = a.token_logits != nullptr;
  const bool ent = a.tau != nullptr, wl = a.logits_out != nullptr;
  if (ent && (!logits || wl || selects)) return hipErrorInvalidValue;
  if (wl && logits) return hipErrorInvalidValue;
  if (a.logits_slots && (d.dtype != kBF16 || a.logits_tm || (!wl && !logits) || a.window))
    return hipErrorInvalidValue;
  if (ent && !(a.alpha_m1 > 0.f && a.alpha_m1 <= 1.f && a.beta >= 1.f)) return hipErrorInvalidValue;
  const bool sliced = a.sl.NB > 0;
  if (sliced && (a.unit != kToken || d.dtype != kBF16 || selects || a.sel_idx || a.window || ent ||
                 wl || !logits || !a.logits_tm || a.logits_slots || a.sub_log2 < 0 ||
                 a.sub_log2 > 3 || a.S != (a.sl.NB << a.sub_log2) || !a.sl.scores || !a.sl.mm ||
                 !a.sl.above || !a.sl.ccount || !a.sl.cand))
    return hipErrorInvalidValue;
  // chunks of 16 rows a wave holds in one split: E pages of P / 16 chunks,
  // or E listed tokens / 16 (sliced: the expected kept units of a range)
  const int64_t nch = a.unit == kPage ? (int64_t)a.E * (d.P / 16) : ((int64_t)a.E + 15) / 16;
  const int64_t cpw = (nch + kAttendWaves - 1) / kAttendWaves;
  const bool ok = dispatch_tdg(d.dtype, d.D, d.G, [&](auto t, auto dd, auto gg) {
    using T = decltype(t);
    constexpr int D = decltype(dd)::value;
    constexpr int G = decltype(gg)::value;
    constexpr int NT = kAttendWaves * 64;
    if constexpr (std::is_same<T, float>::value) {
      attend_f32_kernel<D, G><<<grid, NT, 0, st>>>(a);
    } else if (selects) {
      // the in-kernel top-k feeds softmax attention, or (logits only) the
      // kept tokens' logits that entmax attention later reads
      auto go = [&](auto sel) {
        constexpr int SEL = decltype(sel)::value;
        if (wl) go_mfma<D, G, false, SEL, kWLogits>(a, grid, st, cpw);
        else go_mfma<D, G, false, SEL, kWSoftmax>(a, grid, st, cpw);
      };
      switch (select_mode(d.max_pages)) {
        case kBlock4: go(std::integral_constant<int, kBlock4>{}); break;
        case kBlock8: go(std::integral_constant<int, kBlock8>{}); break;
        default: go(std::integral_constant<int, kBlock32>{}); break;
      }
    } else if (sliced) {
      go_mfma<D, G, true, kSliced, kWSoftmax>(a, grid, st, cpw);
    } else if (wl) {
      go_mfma<D, G, false, kListed, kWLogits>(a, grid, st, cpw);
    } else if (logits && ent) {
      go_mfma<D, G, true, kListed, kWEntmax>(a, grid, st, cpw);
    } else if (logits) {
      go_mfma<D, G, true, kListed, kWSoftmax>(a, grid, st, cpw);
    } else {
      go_mfma<D, G, false, kListed, kWSoftmax>(a, grid, st, cpw);
    }
  });
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t st) {
  const int bh = a.d.B * a.d.Hq;
  if (a.S_known > a.S_max) return hipErrorInvalidValue;
  if (a.d.D == 64)
    merge_splits_kernel<64><<<bh, 256, 0, st>>>(a);
  else
    merge_splits_kernel<128><<<bh, 256, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace sdkv
