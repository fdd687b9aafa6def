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
// hi = max(U - local, lo).  The top-k list is ascending and its ids are
// distinct, so the ids below lo can only be its first lo entries and the
// ids at or above hi only its last U - hi entries: counting those two short
// stretches gives i0 (ids < lo) and i1 (ids < hi), and the union in
// ascending order is [0, lo), then entries i0 .. i1 - 1 of the list, then
// [hi, U).  Blocks (b, g, c) write output positions [c * kStructChunk,
// (c + 1) * kStructChunk), each recounting i0 and i1; every load is issued
// unconditionally with a clamped index, so a thread keeps all of its loads
// in flight.
#include "topk.h"

namespace sdkv {

constexpr int kStructThreads = 256;
constexpr int kStructPer = 16;  // output positions per thread
constexpr int kStructChunk = kStructThreads * kStructPer;

// Number of entries of list[from .. from + m) that are < x (m >= 0, list
// entries in range), summed over the block.
__device__ __forceinline__ int block_count_below(const int32_t* list, int from, int m, int x,
                                                 int* s_red) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int UN = 8;
  int c = 0;
  for (int base = 0; base < m; base += kStructThreads * UN) {
    int v[UN];
#pragma unroll
    for (int u = 0; u < UN; ++u) v[u] = list[from + min(base + u * kStructThreads + tid, m - 1)];
#pragma unroll
    for (int u = 0; u < UN; ++u) c += (base + u * kStructThreads + tid < m && v[u] < x) ? 1 : 0;
  }
  c = (int)wave_sum((uint32_t)c);
  if (lane == 0) s_red[wave] = c;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int w = 0; w < kStructThreads / 64; ++w) t += s_red[w];
  __syncthreads();
  return t;
}

__global__ __launch_bounds__(kStructThreads) void structure_kernel(StructArgs a) {
  __shared__ int s_red[kStructThreads / 64];
  const int BG = a.d.B * a.d.Hkv;
  const int bg = blockIdx.x % BG, chunk = blockIdx.x / BG, b = bg / a.d.Hkv;
  const int tid = threadIdx.x;
  const int n = clamp_len(a.seq_lens[b], a.d.max_seq);
  const int U = a.unit == kPage ? (n + a.d.P - 1) / a.d.P : n;
  int32_t* out = a.sel_idx + (int64_t)bg * a.cap;
  const int p0 = chunk * kStructChunk;
  if (a.kind == kWindow) {
    const int k = min(keep_count_dev(U, a.R_ppm), a.cap);
#pragma unroll
    for (int u = 0; u < kStructPer; ++u) {
      const int i = p0 + u * kStructThreads + tid;
      if (i < k) out[i] = U - k + i;
    }
    if (chunk == 0 && tid == 0) a.sel_count[bg] = k;
    return;
  }
  const int lo = min(a.init_units, U);
  const int hi = max(U - a.local_units, lo);
  const int kc = max(0, min(a.topk_count[bg], a.topk_stride));
  const int32_t* top = a.topk_idx + (int64_t)bg * a.topk_stride;
  const int head = min(lo, kc), tail = min(U - hi, kc);
  const int i0 = block_count_below(top, 0, head, lo, s_red);
  const int i1 = kc - (tail - block_count_below(top, kc - tail, tail, hi, s_red));
  const int mid = i1 - i0;
  const int total = min(lo + mid + (U - hi), a.cap);
  int v[kStructPer];
#pragma unroll
  for (int u = 0; u < kStructPer; ++u) {
    const int i = p0 + u * kStructThreads + tid;
    v[u] = kc > 0 ? top[max(0, min(i0 + i - lo, kc - 1))] : 0;
  }
#pragma unroll
  for (int u = 0; u < kStructPer; ++u) {
    const int i = p0 + u * kStructThreads + tid;
    if (i < total) out[i] = i < lo ? i : (i < lo + mid ? v[u] : hi + (i - lo - mid));
  }
  if (chunk == 0 && tid == 0) a.sel_count[bg] = total;
}

hipError_t launch_structure(const StructArgs& a, hipStream_t st) {
  if (a.cap < 1 || (a.kind != kWindow && a.kind != kInitLocalTopk)) return hipErrorInvalidValue;
  if (a.kind == kInitLocalTopk && (!a.topk_idx || !a.topk_count || a.topk_stride < 1))
    return hipErrorInvalidValue;
  const int chunks = (a.cap + kStructChunk - 1) / kStructChunk;
  structure_kernel<<<a.d.B * a.d.Hkv * chunks, kStructThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace sdkv
