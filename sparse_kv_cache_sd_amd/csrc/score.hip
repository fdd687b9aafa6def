// Stage 1a: query-aware scoring of KV units.
//
// Page unit: an upper bound on each page's largest logit from the page's
// channel-wise key minima and maxima ("Where Activation Sparsity and KV-Cache
// Sparsity Cross in LLM Decoding", cards view, EntmaxKV abstract: pages are
// ranked from light statistics before they are loaded).  For one head,
// sum_c max(q_c kmin_c, q_c kmax_c) = sum_c q_c * (q_c >= 0 ? kmax_c : kmin_c)
// because kmin_c <= kmax_c, and rounding is monotone, so the selected product
// is also the larger one in floating point.  The group's score is the max over
// its G query heads.  The statistics are kept per sequence in logical page
// order, so scoring streams them without a block-table lookup.  A page's
// bound pair is read by LPR = d/8 consecutive lanes, 8 channels (16 B of
// bf16) each; partial sums are reduced with DPP row moves, and every lane
// issues the loads of kScoreIters pages at once, before the sequence length
// is known.
//
// In every kernel here the loads are issued unconditionally (indexes clamped,
// rows that do not count read a valid row and are masked afterwards): a load
// under a branch makes the compiler wait for every outstanding load at the
// join, which would serialise the memory round trips.
//
// Token unit: the exact logits scale * q.K of every valid key, kept for the
// attention pass, and their max over the group ("... list view", Abstract:
// attention-scored KV selection reads every key once).  For bf16 the 16-row
// chunks go through the matrix cores exactly as in the attention kernel
// (S^T = K Q^T with mfma 16x16x32); for fp32 the vector path is used.
#include "topk.h"

namespace sdkv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int kScoreThreads = 256;
constexpr int kScoreIters = 2;
constexpr int kTokenIters = 2;  // 16-token chunks per wave, bf16 token scorer

template <typename T, int D>
constexpr int score_rows_per_block() {
  return (kScoreThreads / 64) * kScoreIters * (64 / (D / 8));
}

template <typename T, int D, int G>
__global__ __launch_bounds__(kScoreThreads) void score_pages_kernel(
    const T* __restrict__ q, const T* __restrict__ bounds,
    const int32_t* __restrict__ seq_lens, float* __restrict__ scores, Dims d) {
  constexpr int LPR = D / 8;
  constexpr int RPW = 64 / LPR;
  constexpr int IT = kScoreIters;
  constexpr int PPB = score_rows_per_block<T, D>();
  const GroupBlock gb = group_block(d.B * d.Hkv);
  const int g = gb.bg % d.Hkv, b = gb.bg / d.Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane / LPR, cl = lane % LPR;
  const int u0 = gb.j * PPB;
  float qv[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
    load8(q + ((int64_t)b * d.Hq + g * G + h) * D + cl * 8, qv[h]);

  // Rows past a sequence's pages are not read.  With one sequence the loads
  // go out before its length is known (the length's round trip then
  // overlaps them, and nothing is skipped but the last block's tail); in a
  // batch of ragged sequences the length is read first, so blocks past the
  // end stop and rows past it re-read the last one.
  int rows = d.max_pages;
  if (d.B > 1) {
    const int nb = clamp_len(seq_lens[b], d.max_seq);
    rows = (nb + d.P - 1) / d.P;
    if (u0 >= rows) return;
  }
  // statistics are stored in logical page order: no block-table lookup
  const T* bnd = bounds + ((int64_t)b * d.Hkv + g) * d.max_pages * 2 * D + cl * 8;
  Raw8<T> lo_w[IT], hi_w[IT];
  int uu[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    uu[it] = u0 + (wave * IT + it) * RPW + sub;
    const int uc = min(uu[it], rows - 1);
    lo_w[it] = load_raw8(bnd + (int64_t)uc * 2 * D);
    hi_w[it] = load_raw8(bnd + (int64_t)uc * 2 * D + D);
  }
  __builtin_amdgcn_sched_barrier(0);  // all loads issue before the first use
  const int n = clamp_len(seq_lens[b], d.max_seq);
  const int U = (n + d.P - 1) / d.P;
  float* out = scores + ((int64_t)b * d.Hkv + g) * d.max_pages;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    float lo[8], hi[8];
    widen8(lo_w[it], lo);
    widen8(hi_w[it], hi);
    float best = -INFINITY;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) acc = fmaf(qv[h][c], qv[h][c] >= 0.f ? hi[c] : lo[c], acc);
      acc = group_sum<LPR>(acc);
      best = fmaxf(best, acc * d.scale);
    }
    if (uu[it] < U && cl == 0) out[uu[it]] = best;
  }
}

// bf16 page scorer on the matrix cores.  The bound of one head is a dense
// contraction over the 2d channels of the stored [kmin | kmax] row:
//   sum_c q_c * (q_c >= 0 ? kmax_c : kmin_c)
//     = sum_c min(q_c, 0) kmin_c + sum_c max(q_c, 0) kmax_c,
// so with Q' = [min(q, 0) | max(q, 0)] (exact in bf16) the scores of 16 pages
// and the 16 (padded) heads of a group are one 16x16 tile of Q' R^T, R the
// pages' bound rows: 2d / 32 mfma 16x16x32 steps.  Q' is the A operand (lane
// (h, quad) holds Q'[h][32 s + 8 quad .. +7]), the bound rows the B operand
// (lane (u, quad) loads 16 bytes of page u's row), and the result lane
// (u, quad) holds heads 4 quad .. 4 quad + 3 of page u, so the max over the
// group needs at most one lane exchange (G = 8).  Each wave scores
// kPageTiles tiles of 16 pages, all loads issued before the first product.
// Used for bf16 groups of more than four heads.
constexpr int kPageTiles = 1;

template <int D, int G>
__global__ __launch_bounds__(kScoreThreads) void score_pages_mfma_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ bounds,
    const int32_t* __restrict__ seq_lens, float* __restrict__ scores, Dims d) {
  constexpr int KS = 2 * D / 32;  // steps over the 2d channels
  constexpr int NW = kScoreThreads / 64, IT = kPageTiles;
  constexpr int PPB = NW * IT * 16;
  static_assert(G <= 8, "at most two quads of heads");
  const GroupBlock gb = group_block(d.B * d.Hkv);
  const int g = gb.bg % d.Hkv, b = gb.bg / d.Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, quad = lane >> 4;
  const int u0 = gb.j * PPB + wave * IT * 16;

  // rows past a sequence's pages: as in score_pages_kernel (re-read the
  // last row in a batch, whose lengths are read first)
  int rows = d.max_pages;
  if (d.B > 1) rows = max((clamp_len(seq_lens[b], d.max_seq) + d.P - 1) / d.P, 1);
  // statistics are stored in logical page order: no block-table lookup
  const bf16_t* bnd = bounds + ((int64_t)b * d.Hkv + g) * d.max_pages * 2 * D + 8 * quad;
  u32x4_t rw[IT][KS];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int uc = min(u0 + 16 * it + col, rows - 1);
#pragma unroll
    for (int s = 0; s < KS; ++s)
      rw[it][s] = *reinterpret_cast<const u32x4_t*>(bnd + (int64_t)uc * 2 * D + 32 * s);
  }
  u32x4_t qw[KS];
  {
    const bf16_t* qrow = q + ((int64_t)b * d.Hq + g * G + min(col, G - 1)) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qw[s] = *reinterpret_cast<const u32x4_t*>(qrow + (32 * s + 8 * quad) % D);
  }
  __builtin_amdgcn_sched_barrier(0);  // all loads issue before the first use
  // A operand: the negative parts against kmin (first d channels), the
  // positive parts against kmax; padded heads are zero.
  bf16x8_t qop[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const bool neg_half = 32 * s < D;
    u32x4_t w = qw[s];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // per 16-bit half: keep it when its sign matches the half (sign set
      // for min(q, 0), clear for max(q, 0)), else zero
      const uint32_t sgn = w[i] & 0x80008000u;
      const uint32_t m = (sgn >> 15) * 0xFFFFu;  // 0xFFFF per half with its sign set
      w[i] &= neg_half ? m : ~m;
    }
    if (col >= G) w = u32x4_t{0u, 0u, 0u, 0u};
    qop[s] = __builtin_bit_cast(bf16x8_t, w);
  }
  const int n = clamp_len(seq_lens[b], d.max_seq);
  const int U = (n + d.P - 1) / d.P;
  float* out = scores + ((int64_t)b * d.Hkv + g) * d.max_pages;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    float4_t st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s)
      st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qop[s], __builtin_bit_cast(bf16x8_t, rw[it][s]),
                                                    st, 0, 0, 0);
    float best = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (4 * quad + r < G) best = fmaxf(best, st[r] * d.scale);
    if constexpr (G > 4) best = max_xor16(best);
    const int u = u0 + 16 * it + col;
    if (quad == 0 && u < U) out[u] = best;
  }
}

// Block-wide min and max of the per-lane key ranges, stored as partial x of
// bg (nx partials per bg): mm[(bg * nx + x) * 2 + {0, 1}].
__device__ __forceinline__ void block_partial_minmax(uint32_t* mm, uint32_t mn, uint32_t mx,
                                                     int64_t bg, int x, int nx) {
  __shared__ uint32_t s_mm[2][kScoreThreads / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  mn = wave_umin(mn);
  mx = wave_umax(mx);
  if (lane == 0) { s_mm[0][wave] = mn; s_mm[1][wave] = mx; }
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int w = 1; w < kScoreThreads / 64; ++w) {
      mn = min(mn, s_mm[0][w]);
      mx = max(mx, s_mm[1][w]);
    }
    mm[(bg * nx + x) * 2] = mn;
    mm[(bg * nx + x) * 2 + 1] = mx;
  }
}

// fp32 token scorer (vector FMAs).
template <int D, int G>
__global__ __launch_bounds__(kScoreThreads) void score_tokens_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k_pages,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens,
    float* __restrict__ scores, float* __restrict__ logits, uint32_t* __restrict__ mm, Dims d,
    int tm) {
  constexpr int LPR = D / 8;
  constexpr int RPW = 64 / LPR;
  constexpr int IT = kScoreIters;
  constexpr int TPB = score_rows_per_block<float, D>();
  const int BG = d.B * d.Hkv;
  const GroupBlock gb = group_block(BG);
  const int g = gb.bg % d.Hkv, b = gb.bg / d.Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane / LPR, cl = lane % LPR;
  const int n = clamp_len(seq_lens[b], d.max_seq);
  const int t0 = gb.j * TPB;
  if (t0 >= n) return;

  float qv[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
    load8(q + ((int64_t)b * d.Hq + g * G + h) * D + cl * 8, qv[h]);

  Raw8<float> kw[IT];
  bool ok[IT];
  int tt[IT], phys[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    tt[it] = t0 + (wave * IT + it) * RPW + sub;
    const int lp = min(tt[it] / d.P, d.max_pages - 1);
    phys[it] = block_table[(int64_t)b * d.max_pages + lp];
  }
  const float* qrow0 = q + ((int64_t)b * d.Hq + g * G) * D + cl * 8;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    ok[it] = tt[it] < n && phys[it] >= 0 && phys[it] < d.num_pages;
    const int lp = tt[it] / d.P;
    kw[it] = load_raw8(ok[it] ? k_pages + (((int64_t)phys[it] * d.Hkv + g) * d.P +
                                           (tt[it] - lp * d.P)) * D + cl * 8
                              : qrow0);
  }
  __builtin_amdgcn_sched_barrier(0);
  float* sc = scores + ((int64_t)b * d.Hkv + g) * d.max_seq;
  uint32_t kmn = 0xFFFFFFFFu, kmx = 0u;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    float kv[8];
    widen8(kw[it], kv);
    float best = -INFINITY, mine = 0.f;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) acc = fmaf(qv[h][c], kv[c], acc);
      const float s = group_sum<LPR>(acc) * d.scale;
      best = fmaxf(best, s);
      if (h == cl) mine = s;
    }
    const int t = tt[it];
    if (t < n) {
      if (!ok[it]) { best = -3.0e38f; mine = -3.0e38f; }
      if (cl < G) {
        const int64_t at = tm ? (((int64_t)b * d.Hkv + g) * d.max_seq + t) * G + cl
                              : ((int64_t)b * d.Hq + g * G + cl) * d.max_seq + t;
        logits[at] = mine;
      }
      if (cl == 0) sc[t] = best;
      kmn = min(kmn, order_key(best));
      kmx = max(kmx, order_key(best));
    }
  }
  if (mm) block_partial_minmax(mm, kmn, kmx, gb.bg, gb.j, (d.max_seq + TPB - 1) / TPB);
}

// bf16 token scorer on the matrix cores: each wave scores kTokenIters chunks
// of 16 consecutive tokens (16 | P, so a chunk lies in one page and its rows
// are contiguous in the page tile).
template <int D, int G>
__global__ __launch_bounds__(kScoreThreads) void score_tokens_mfma_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k_pages,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens,
    float* __restrict__ scores, float* __restrict__ logits, uint32_t* __restrict__ mm, Dims d,
    int tm) {
  // token-major logits: a chunk's 16 x G values go through LDS so that they
  // leave as whole consecutive pieces (16 G floats per chunk)
  __shared__ __align__(16) float s_lg[kScoreThreads / 64][16 * G];
  constexpr int KS = D / 32;
  constexpr int IT = kTokenIters;
  constexpr int NW = kScoreThreads / 64;
  constexpr int TPB = NW * IT * 16;
  const int BG = d.B * d.Hkv;
  const GroupBlock gb = group_block(BG);
  const int g = gb.bg % d.Hkv, b = gb.bg / d.Hkv;
  const int lane = threadIdx.x & 63;
  // the wave index as a wave-uniform value, so that each chunk's block-table
  // entry is a scalar load (the K loads wait on it: 58.5 -> 57.2 us at 128K
  // tokens against a vector load queued behind the q loads)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row = lane & 15, quad = lane >> 4;
  const int n = clamp_len(seq_lens[b], d.max_seq);
  const int t0 = gb.j * TPB;
  if (t0 >= n) return;

  bf16x8_t qop[KS];
  {
    const bf16_t* qrow = q + ((int64_t)b * d.Hq + g * G + row) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      uint4 w = make_uint4(0u, 0u, 0u, 0u);
      if (row < G) w = *reinterpret_cast<const uint4*>(qrow + 32 * s + 8 * quad);
      qop[s] = __builtin_bit_cast(bf16x8_t, w);
    }
  }
  u32x4_t kv[IT][KS];
  bool page_ok[IT];
  int tc[IT], phys[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    tc[it] = t0 + (wave * IT + it) * 16;
    const int lp = min(tc[it] / d.P, d.max_pages - 1);
    phys[it] = block_table[(int64_t)b * d.max_pages + lp];
  }
  const bf16_t* qrow0 = q + ((int64_t)b * d.Hq + g * G) * D;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int t = tc[it] + row;
    const int lp = tc[it] / d.P;
    page_ok[it] = tc[it] < n && phys[it] >= 0 && phys[it] < d.num_pages;
    const bf16_t* kr = page_ok[it] && t < n
                           ? k_pages + (((int64_t)phys[it] * d.Hkv + g) * d.P + (t - lp * d.P)) * D
                           : qrow0;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      kv[it][s] = *reinterpret_cast<const u32x4_t*>(kr + 32 * s + 8 * quad);
  }
  __builtin_amdgcn_sched_barrier(0);
  float* sc = scores + ((int64_t)b * d.Hkv + g) * d.max_seq;
  float* lg = logits + ((int64_t)b * d.Hq + g * G + min(row, G - 1)) * d.max_seq;
  float* lg_tm = logits + ((int64_t)b * d.Hkv + g) * d.max_seq * G;
  uint32_t kmn = 0xFFFFFFFFu, kmx = 0u;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    if (tc[it] >= n) continue;
    float4_t st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s)
      st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kv[it][s]), qop[s],
                                                    st, 0, 0, 0);
    // lane (row = head, quad) holds tokens tc + 4 quad + r: four consecutive
    // logits of one head, written with one 16-byte store when all are valid
    const int t4 = tc[it] + 4 * quad;
    float4_t xs, bs;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      xs[r] = page_ok[it] ? st[r] * d.scale : -3.0e38f;
      bs[r] = group_max<16>(row < G ? xs[r] : -INFINITY);
      if (t4 + r < n) {
        kmn = min(kmn, order_key(bs[r]));
        kmx = max(kmx, order_key(bs[r]));
      }
    }
    if (tm) {
      // lane (row = head, quad) holds tokens 4 quad + r: stage [token][head],
      // then lane i writes floats 4i .. 4i + 3 of the chunk (G >= 4: part of
      // one token's G logits) or float i (G < 4), tokens past n left out
      float* st_w = s_lg[wave];
      if (row < G) {
#pragma unroll
        for (int r = 0; r < 4; ++r) st_w[(4 * quad + r) * G + row] = xs[r];
      }
      __builtin_amdgcn_wave_barrier();
      if constexpr (G >= 4) {
        if (lane < 4 * G && tc[it] + (4 * lane) / G < n)
          *reinterpret_cast<float4_t*>(lg_tm + (int64_t)tc[it] * G + 4 * lane) =
              *reinterpret_cast<const float4_t*>(st_w + 4 * lane);
      } else {
        if (lane < 16 * G && tc[it] + lane / G < n)
          lg_tm[(int64_t)tc[it] * G + lane] = st_w[lane];
      }
      __builtin_amdgcn_wave_barrier();
      if ((d.max_seq & 3) == 0 && t4 + 3 < n) {
        if (row == 0) *reinterpret_cast<float4_t*>(sc + t4) = bs;
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (t4 + r < n && row == 0) sc[t4 + r] = bs[r];
      }
    } else if ((d.max_seq & 3) == 0 && t4 + 3 < n) {  // rows are 16-byte aligned
      if (row < G) *reinterpret_cast<float4_t*>(lg + t4) = xs;
      if (row == 0) *reinterpret_cast<float4_t*>(sc + t4) = bs;
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (t4 + r < n) {
          if (row < G) lg[t4 + r] = xs[r];
          if (row == 0) sc[t4 + r] = bs[r];
        }
      }
    }
  }
  if (mm) block_partial_minmax(mm, kmn, kmx, gb.bg, gb.j, (d.max_seq + TPB - 1) / TPB);
}

int score_units_per_block(int dtype, int D) {
  if (dtype == kBF16) return (kScoreThreads / 64) * kTokenIters * 16;
  return D == 64 ? score_rows_per_block<float, 64>() : score_rows_per_block<float, 128>();
}

hipError_t launch_score(const ScoreArgs& a, hipStream_t st) {
  const Dims& d = a.d;
  const bool ok = dispatch_tdg(d.dtype, d.D, d.G, [&](auto t, auto dd, auto gg) {
    using T = decltype(t);
    constexpr int D = decltype(dd)::value;
    constexpr int G = decltype(gg)::value;
    if (a.unit == kPage) {
      // bf16 groups of more than 4 heads go to the matrix cores (their 8
      // sign-selected products per channel cost the vector path more than
      // its loads); smaller groups stay on the vector path, which measured
      // faster there
      if constexpr (std::is_same<T, float>::value || G <= 4) {
        constexpr int R = score_rows_per_block<T, D>();
        const dim3 grid((d.max_pages + R - 1) / R * d.Hkv * d.B);
        score_pages_kernel<T, D, G><<<grid, kScoreThreads, 0, st>>>(
            static_cast<const T*>(a.q), static_cast<const T*>(a.bounds), a.seq_lens,
            a.unit_scores, d);
      } else {
        constexpr int R = (kScoreThreads / 64) * kPageTiles * 16;
        const dim3 grid((d.max_pages + R - 1) / R * d.Hkv * d.B);
        score_pages_mfma_kernel<D, G><<<grid, kScoreThreads, 0, st>>>(
            static_cast<const bf16_t*>(a.q), static_cast<const bf16_t*>(a.bounds), a.seq_lens,
            a.unit_scores, d);
      }
    } else if constexpr (std::is_same<T, float>::value) {
      constexpr int R = score_rows_per_block<T, D>();
      const dim3 grid((d.max_seq + R - 1) / R * d.Hkv * d.B);
      score_tokens_f32_kernel<D, G><<<grid, kScoreThreads, 0, st>>>(
          static_cast<const float*>(a.q), static_cast<const float*>(a.k_pages), a.block_table,
          a.seq_lens, a.unit_scores, a.token_logits, a.score_mm, d, a.logits_tm);
    } else {
      constexpr int R = (kScoreThreads / 64) * kTokenIters * 16;
      const dim3 grid((d.max_seq + R - 1) / R * d.Hkv * d.B);
      score_tokens_mfma_kernel<D, G><<<grid, kScoreThreads, 0, st>>>(
          static_cast<const bf16_t*>(a.q), static_cast<const bf16_t*>(a.k_pages), a.block_table,
          a.seq_lens, a.unit_scores, a.token_logits, a.score_mm, d, a.logits_tm);
    }
  });
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace sdkv
