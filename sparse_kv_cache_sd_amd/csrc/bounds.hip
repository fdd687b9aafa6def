// Per-page key statistics: channel-wise min and max over a page's valid
// tokens, the light page statistics that page scoring reads before any page
// is loaded ("Where Activation Sparsity and KV-Cache Sparsity Cross in LLM
// Decoding", cards view, EntmaxKV abstract).  A setup step, not part of the
// timed decode step.
#include "device.h"

namespace sdkv {

// Layout of the result: [B][H_kv][max_pages][2][d] in logical page order, so
// that scoring streams a sequence's statistics without the block table.
// grid (max_pages, B), block 256: one block per logical page of a sequence,
// one thread per (KV head, channel) pair, looping over the page's valid rows.
constexpr int kBoundsThreads = 256;

template <typename T>
__global__ __launch_bounds__(kBoundsThreads) void page_bounds_kernel(
    const T* __restrict__ k_pages, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, T* __restrict__ bounds, Dims d) {
  const int u = blockIdx.x, b = blockIdx.y;
  const int n = clamp_len(seq_lens[b], d.max_seq);
  const int U = (n + d.P - 1) / d.P;
  if (u >= U) return;
  const int phys = block_table[(int64_t)b * d.max_pages + u];
  if (phys < 0 || phys >= d.num_pages) return;
  const int valid = min(d.P, n - u * d.P);
  for (int idx = threadIdx.x; idx < d.Hkv * d.D; idx += kBoundsThreads) {
    const int g = idx / d.D, c = idx - g * d.D;
    const T* col = k_pages + ((int64_t)phys * d.Hkv + g) * d.P * d.D + c;
    float lo = to_f(col[0]), hi = lo;
    for (int t = 1; t < valid; ++t) {
      const float v = to_f(col[(int64_t)t * d.D]);
      lo = fminf(lo, v);
      hi = fmaxf(hi, v);
    }
    T* dst = bounds + (((int64_t)b * d.Hkv + g) * d.max_pages + u) * 2 * d.D + c;
    dst[0] = from_f<T>(lo);
    dst[d.D] = from_f<T>(hi);
  }
}

hipError_t launch_page_bounds(const BoundsArgs& a, hipStream_t st) {
  const dim3 grid(a.d.max_pages, a.d.B);
  if (a.d.dtype == kF32) {
    page_bounds_kernel<float><<<grid, kBoundsThreads, 0, st>>>(
        static_cast<const float*>(a.k_pages), a.block_table, a.seq_lens,
        static_cast<float*>(a.bounds), a.d);
  } else {
    page_bounds_kernel<bf16_t><<<grid, kBoundsThreads, 0, st>>>(
        static_cast<const bf16_t*>(a.k_pages), a.block_table, a.seq_lens,
        static_cast<bf16_t*>(a.bounds), a.d);
  }
  return hipGetLastError();
}

}  // namespace sdkv
