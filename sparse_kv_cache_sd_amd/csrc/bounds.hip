// Per-page key statistics: channel-wise min and max over a page's valid
// tokens, the light page statistics that page scoring reads before any page
// is loaded ("Where Activation Sparsity and KV-Cache Sparsity Cross in LLM
// Decoding", cards view, EntmaxKV abstract).  A setup step, not part of the
// timed decode step, in three forms:
//   * every page of every sequence;
//   * a listed subset of (sequence, logical page) pairs, each recomputed over
//     its valid rows;
//   * an append: the tokens that joined each sequence since the last update
//     are folded into their pages' bounds, O(d) per appended token and KV
//     head; a page that an appended token opens starts from that token.
// min and max are exact in any order, so all three give the same bits.
#include "device.h"

namespace sdkv {

// Layout of the result: [B][H_kv][max_pages][2][d] in logical page order, so
// that scoring streams a sequence's statistics without the block table.
// One block per (sequence, logical page); one thread per (KV head, channel)
// pair, looping over the page's rows (threads of a wave read consecutive
// channels of a row: coalesced).
constexpr int kBoundsThreads = 256;

// Rows [r0, r1) of logical page u of sequence b (physical page phys) folded
// into its bounds; fresh: the bounds start from row r0 instead of the stored
// ones.  r0 < r1.
template <typename T>
__device__ __forceinline__ void fold_page(const T* __restrict__ k_pages, T* __restrict__ bounds,
                                          const Dims& d, int b, int u, int phys, int r0, int r1,
                                          bool fresh) {
  for (int idx = threadIdx.x; idx < d.Hkv * d.D; idx += kBoundsThreads) {
    const int g = idx / d.D, c = idx - g * d.D;
    const T* col = k_pages + ((int64_t)phys * d.Hkv + g) * d.P * d.D + c;
    T* dst = bounds + (((int64_t)b * d.Hkv + g) * d.max_pages + u) * 2 * d.D + c;
    float lo, hi;
    int t = r0;
    if (fresh) {
      lo = hi = to_f(col[(int64_t)t * d.D]);
      ++t;
    } else {
      lo = to_f(dst[0]);
      hi = to_f(dst[d.D]);
    }
    for (; t < r1; ++t) {
      const float v = to_f(col[(int64_t)t * d.D]);
      lo = fminf(lo, v);
      hi = fmaxf(hi, v);
    }
    dst[0] = from_f<T>(lo);
    dst[d.D] = from_f<T>(hi);
  }
}

// Physical page of logical page u of sequence b, or -1 when the entry is
// outside the pool (such a page is never read, so its bounds are not kept).
__device__ __forceinline__ int phys_page(const int32_t* __restrict__ block_table, const Dims& d,
                                         int b, int u) {
  const int phys = block_table[(int64_t)b * d.max_pages + u];
  return (phys < 0 || phys >= d.num_pages) ? -1 : phys;
}

// Every page: grid (max_pages, B).
template <typename T>
__global__ __launch_bounds__(kBoundsThreads) void page_bounds_kernel(
    const T* __restrict__ k_pages, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, T* __restrict__ bounds, Dims d) {
  const int u = blockIdx.x, b = blockIdx.y;
  const int n = clamp_len(seq_lens[b], d.max_seq);
  if (u * d.P >= n) return;
  const int phys = phys_page(block_table, d, b, u);
  if (phys < 0) return;
  fold_page(k_pages, bounds, d, b, u, phys, 0, min(d.P, n - u * d.P), true);
}

// Listed pages: block i recomputes pair pages[i] = (sequence, logical page);
// pairs outside the batch or past the sequence's last page are skipped.
template <typename T>
__global__ __launch_bounds__(kBoundsThreads) void page_bounds_list_kernel(
    const T* __restrict__ k_pages, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ pages,
    T* __restrict__ bounds, Dims d) {
  const int b = pages[2 * (int64_t)blockIdx.x], u = pages[2 * (int64_t)blockIdx.x + 1];
  if (b < 0 || b >= d.B || u < 0 || u >= d.max_pages) return;
  const int n = clamp_len(seq_lens[b], d.max_seq);
  if (u * d.P >= n) return;
  const int phys = phys_page(block_table, d, b, u);
  if (phys < 0) return;
  fold_page(k_pages, bounds, d, b, u, phys, 0, min(d.P, n - u * d.P), true);
}

// Append: sequence b gained the tokens [n_b - a_b, n_b) (a_b = appended[b],
// clamped to [0, min(n_b, max_appended)]); grid (pages_per_seq, B), block j
// takes the j-th page those tokens touch.  Rows before the first appended one are already in the
// stored bounds; a page whose first appended row is row 0 starts fresh.
template <typename T>
__global__ __launch_bounds__(kBoundsThreads) void page_bounds_append_kernel(
    const T* __restrict__ k_pages, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ appended,
    T* __restrict__ bounds, Dims d, int max_appended) {
  const int b = blockIdx.y;
  const int n = clamp_len(seq_lens[b], d.max_seq);
  const int a = min(max(appended[b], 0), min(n, max_appended));
  if (a == 0) return;
  const int first = n - a;
  const int u = first / d.P + (int)blockIdx.x;
  if (u * d.P >= n) return;
  const int phys = phys_page(block_table, d, b, u);
  if (phys < 0) return;
  const int r0 = max(first - u * d.P, 0);
  fold_page(k_pages, bounds, d, b, u, phys, r0, min(d.P, n - u * d.P), r0 == 0);
}

template <typename T>
static hipError_t launch_bounds_t(const BoundsArgs& a, hipStream_t st) {
  const T* k = static_cast<const T*>(a.k_pages);
  T* out = static_cast<T*>(a.bounds);
  if (a.pages) {
    if (a.n_pages > 0)
      page_bounds_list_kernel<T><<<a.n_pages, kBoundsThreads, 0, st>>>(
          k, a.block_table, a.seq_lens, a.pages, out, a.d);
  } else if (a.appended) {
    // at most ceil(max_appended / P) + 1 pages are touched per sequence
    const int per = (a.max_appended + a.d.P - 1) / a.d.P + 1;
    page_bounds_append_kernel<T><<<dim3(min(per, a.d.max_pages), a.d.B), kBoundsThreads, 0, st>>>(
        k, a.block_table, a.seq_lens, a.appended, out, a.d, a.max_appended);
  } else {
    page_bounds_kernel<T><<<dim3(a.d.max_pages, a.d.B), kBoundsThreads, 0, st>>>(
        k, a.block_table, a.seq_lens, out, a.d);
  }
  return hipGetLastError();
}

hipError_t launch_page_bounds(const BoundsArgs& a, hipStream_t st) {
  return a.d.dtype == kF32 ? launch_bounds_t<float>(a, st) : launch_bounds_t<bf16_t>(a, st);
}

}  // namespace sdkv
