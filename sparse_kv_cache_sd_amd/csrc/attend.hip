// Stage 2: split-K attention over the kept units, then the log-sum-exp merge.
//
// Dense and sparse decoding share this kernel ("Where Activation Sparsity and
// KV-Cache Sparsity Cross in LLM Decoding", list view, Abstract); a dense call
// is the same kernel with every unit kept.  Attention runs over the tokens of
// the kept blocks only ("SparDA ..." summary, Section 3.1).
//
// Work: block (split j, KV head g, sequence b) takes kept units
// [j*E, min((j+1)*E, count)) of its list; a page unit expands to its P rows
// (rows past n_b are skipped), a token unit is one row.  Each row is read by
// LPR = d/8 lanes, 8 channels each, so one wave covers RPW = 64/LPR rows per
// step and four waves interleave.  Every lane-row keeps its own online
// softmax state (running max m, sum l, weighted sum acc) per query head of
// the group, in the base-2 domain (q is pre-scaled by scale * log2 e).  At
// the end the RPW lane-rows of a wave merge by shuffles, the four waves merge
// through LDS, and the block writes one normalised partial output and its
// log-sum-exp per head; a split with no valid row writes lse = -inf.
// The merge kernel combines the S partials of each head by log-sum-exp.
#include "device.h"

namespace sdkv {

constexpr int kAttendThreads = 256;

template <typename T, int D, int G>
__global__ __launch_bounds__(kAttendThreads) void attend_splitk_kernel(AttendArgs a) {
  constexpr int LPR = D / 8;
  constexpr int RPW = 64 / LPR;
  constexpr int NW = kAttendThreads / 64;
  const Dims& d = a.d;
  const int j = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane / LPR, cl = lane % LPR;
  const int n = clamp_len(a.seq_lens[b], d.max_seq);
  const int U = a.unit == kPage ? (n + d.P - 1) / d.P : n;
  const int64_t bg = (int64_t)b * d.Hkv + g;
  int cnt = U;
  const int32_t* list = nullptr;
  if (a.sel_idx != nullptr) {
    cnt = min(min(a.sel_count[bg], a.k_max), U);
    list = a.sel_idx + bg * a.k_max;
  }
  const int e0 = j * a.E;
  const int e1 = min(cnt, e0 + a.E);
  const int tpe = a.unit == kPage ? d.P : 1;
  const int rows = e1 > e0 ? (e1 - e0) * tpe : 0;
  const bool use_logits = a.token_logits != nullptr;

  const T* qb = static_cast<const T*>(a.q) + ((int64_t)b * d.Hq + g * G) * D + cl * 8;
  const T* kp = static_cast<const T*>(a.k_pages);
  const T* vp = static_cast<const T*>(a.v_pages);
  const float qs = d.scale * kLog2e;
  float qv[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    load8(qb + h * D, qv[h]);
#pragma unroll
    for (int c = 0; c < 8; ++c) qv[h][c] *= qs;
  }

  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[h][c] = 0.f;
  }

  for (int base = wave * RPW; base < rows; base += NW * RPW) {
    const int r = base + sub;
    bool ok = r < rows;
    int t = 0;
    int64_t row_off = 0;
    if (ok) {
      const int e = e0 + r / tpe;
      const int within = r - (r / tpe) * tpe;
      const int uu = list ? list[e] : e;
      if (a.unit == kPage) {
        t = uu * d.P + within;
        ok = uu >= 0 && uu < U && t < n;
      } else {
        t = uu;
        ok = t >= 0 && t < n;
      }
      if (ok) {
        const int lp = t / d.P;
        const int phys = a.block_table[(int64_t)b * d.max_pages + lp];
        ok = phys >= 0 && phys < d.num_pages;
        row_off = (((int64_t)phys * d.Hkv + g) * d.P + (t - lp * d.P)) * D + cl * 8;
      }
    }
    float s[G];
    if (use_logits) {
#pragma unroll
      for (int h = 0; h < G; ++h)
        s[h] = ok ? a.token_logits[((int64_t)b * d.Hq + g * G + h) * d.max_seq + t] * kLog2e : 0.f;
    } else {
      float kv[8];
      if (ok) {
        load8(kp + row_off, kv);
      } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) kv[c] = 0.f;
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float dot = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) dot = fmaf(qv[h][c], kv[c], dot);
#pragma unroll
        for (int o = LPR / 2; o > 0; o >>= 1) dot += __shfl_xor(dot, o, LPR);
        s[h] = dot;
      }
    }
    if (ok) {
      float vv[8];
      load8(vp + row_off, vv);
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

  // Merge the RPW lane-rows of this wave (shuffles across rows of LPR lanes).
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float M = m[h];
#pragma unroll
    for (int o = LPR; o < 64; o <<= 1) M = fmaxf(M, __shfl_xor(M, o));
    const float f = m[h] == -INFINITY ? 0.f : exp2f(m[h] - M);
    l[h] *= f;
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[h][c] *= f;
#pragma unroll
    for (int o = LPR; o < 64; o <<= 1) {
      l[h] += __shfl_xor(l[h], o);
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[h][c] += __shfl_xor(acc[h][c], o);
    }
    m[h] = M;
  }

  // Merge the waves through LDS.
  __shared__ float s_m[NW][G], s_l[NW][G];
  __shared__ float s_acc[NW][G][D];
  if (sub == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int c = 0; c < 8; ++c) s_acc[wave][h][cl * 8 + c] = acc[h][c];
      if (cl == 0) { s_m[wave][h] = m[h]; s_l[wave][h] = l[h]; }
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * D; idx += kAttendThreads) {
    const int h = idx / D, c = idx - h * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, s_m[w][h]);
    float L = 0.f, A = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float f = s_m[w][h] == -INFINITY ? 0.f : exp2f(s_m[w][h] - M);
        L = fmaf(s_l[w][h], f, L);
        A = fmaf(s_acc[w][h][c], f, A);
      }
    }
    const int64_t hs = ((int64_t)b * d.Hq + g * G + h) * a.S + j;
    a.part_o[hs * D + c] = L > 0.f ? A / L : 0.f;
    if (c == 0) a.part_lse[hs] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
  }
}

// One block per (sequence, query head), one thread per channel.
template <int D>
__global__ __launch_bounds__(D) void merge_lse_kernel(const float* __restrict__ part_o,
                                                      const float* __restrict__ part_lse,
                                                      float* __restrict__ out,
                                                      float* __restrict__ lse, int S) {
  const int64_t bh = blockIdx.x;
  const int c = threadIdx.x;
  const float* pl = part_lse + bh * S;
  float M = -INFINITY;
  for (int j = 0; j < S; ++j) M = fmaxf(M, pl[j]);
  if (M == -INFINITY) {
    out[bh * D + c] = 0.f;
    if (c == 0) lse[bh] = -INFINITY;
    return;
  }
  float L = 0.f, A = 0.f;
  for (int j = 0; j < S; ++j) {
    const float w = expf(pl[j] - M);
    L += w;
    A = fmaf(w, part_o[(bh * S + j) * D + c], A);
  }
  out[bh * D + c] = A / L;
  if (c == 0) lse[bh] = M + logf(L);
}

hipError_t launch_attend(const AttendArgs& a, hipStream_t st) {
  const Dims& d = a.d;
  const dim3 grid(a.S, d.Hkv, d.B);
  const bool ok = dispatch_tdg(d.dtype, d.D, d.G, [&](auto t, auto dd, auto gg) {
    using T = decltype(t);
    constexpr int D = decltype(dd)::value;
    constexpr int G = decltype(gg)::value;
    attend_splitk_kernel<T, D, G><<<grid, kAttendThreads, 0, st>>>(a);
  });
  if (!ok) return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int bh = d.B * d.Hq;
  if (d.D == 64)
    merge_lse_kernel<64><<<bh, 64, 0, st>>>(a.part_o, a.part_lse, a.out, a.lse, a.S);
  else
    merge_lse_kernel<128><<<bh, 128, 0, st>>>(a.part_o, a.part_lse, a.out, a.lse, a.S);
  return hipGetLastError();
}

}  // namespace sdkv
