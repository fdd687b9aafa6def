// Structured kept lists: the KV window and the union of initial, local and
// top-k units.
//
// The window keeps the keep_count(r_KV, U) most recent units: the KV-window
// baseline of "Where Activation Sparsity and KV-Cache Sparsity Cross in LLM
// Decoding" (list view, Table 3).  The union keeps the first and the last
// units of the sequence plus the top-k of all its units, the block set of
// "SparDA: Sparse Decoupled Attention ..." (summary, Section 3.1; Appendix A
// writes it as B_init U B_local U f_top(scores, k)).
//
// The forced ranges are [0, lo) and [hi, U) with lo = min(init, U) and
// hi = max(U - local, lo); the top-k list is ascending, so the union in
// ascending order is [0, lo), then the top-k ids in [lo, hi) -- a contiguous
// slice of the list, found by counting its ids below lo and below hi --
// then [hi, U).  Every output position is computed independently.
#include "topk.h"

namespace sdkv {

constexpr int kStructThreads = 256;

__global__ __launch_bounds__(kStructThreads) void structure_kernel(StructArgs a) {
  __shared__ int s_red[2][kStructThreads / 64];
  const int bg = blockIdx.x, b = bg / a.d.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = clamp_len(a.seq_lens[b], a.d.max_seq);
  const int U = a.unit == kPage ? (n + a.d.P - 1) / a.d.P : n;
  int32_t* out = a.sel_idx + (int64_t)bg * a.cap;
  if (a.kind == kWindow) {
    const int k = min(keep_count_dev(U, a.R_ppm), a.cap);
    for (int i = tid; i < k; i += kStructThreads) out[i] = U - k + i;
    if (tid == 0) a.sel_count[bg] = k;
    return;
  }
  const int lo = min(a.init_units, U);
  const int hi = max(U - a.local_units, lo);
  const int kc = max(0, min(a.topk_count[bg], a.topk_stride));
  const int32_t* top = a.topk_idx + (int64_t)bg * a.topk_stride;
  int c_lo = 0, c_hi = 0;
  for (int i = tid; i < kc; i += kStructThreads) {
    const int v = top[i];
    c_lo += v < lo;
    c_hi += v < hi;
  }
  c_lo = (int)wave_sum((uint32_t)c_lo);
  c_hi = (int)wave_sum((uint32_t)c_hi);
  if (lane == 0) { s_red[0][wave] = c_lo; s_red[1][wave] = c_hi; }
  __syncthreads();
  int i0 = 0, i1 = 0;
#pragma unroll
  for (int w = 0; w < kStructThreads / 64; ++w) { i0 += s_red[0][w]; i1 += s_red[1][w]; }
  const int mid = i1 - i0;
  const int total = min(lo + mid + (U - hi), a.cap);
  for (int i = tid; i < total; i += kStructThreads)
    out[i] = i < lo ? i : (i < lo + mid ? top[i0 + i - lo] : hi + (i - lo - mid));
  if (tid == 0) a.sel_count[bg] = total;
}

hipError_t launch_structure(const StructArgs& a, hipStream_t st) {
  if (a.cap < 1 || (a.kind != kWindow && a.kind != kInitLocalTopk)) return hipErrorInvalidValue;
  if (a.kind == kInitLocalTopk && (!a.topk_idx || !a.topk_count || a.topk_stride < 1))
    return hipErrorInvalidValue;
  structure_kernel<<<a.d.B * a.d.Hkv, kStructThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace sdkv
