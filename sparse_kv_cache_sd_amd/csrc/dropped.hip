// Dropped mass delta of the dense softmax, token unit.
//
// "Where Activation Sparsity and KV-Cache Sparsity Cross in LLM Decoding",
// cards view, pre-hoc sparsity abstract: the dropped mass delta -- the dense
// attention probability of the entries left out -- governs the error of
// sparse attention.  In token unit every logit is stored, so delta is one
// more pass over them: for query head h of sequence b,
//   delta = sum_{t not kept} exp(s_t - m) / sum_t exp(s_t - m),
// over the attended tokens t (t < n_b, page block-table entry valid), m the
// max logit.  The dropped tokens are summed directly rather than as one
// minus the kept mass, so a small delta keeps its relative precision.
//
// One 1024-thread block per (sequence, query head); block id
// bg + B * H_kv * (h mod G) as in the other per-head kernels.  The kept list
// of the head's KV head becomes a bitmap in LDS (bits set with LDS atomic
// OR, which gives the same bitmap in any order); the logits are read twice
// (max, then the two sums), eight rounds of loads issued together; every
// sum runs in a fixed order, so delta does not depend on timing.  One block
// per head keeps few bytes in flight per CU, so where the rows are 16-byte
// aligned (max_seq % 4 == 0) a thread reads four consecutive tokens per
// load: they share a page (P is 16 or 64) and a bitmap word.
#include "device.h"

namespace sdkv {

constexpr int kDropThreads = 1024;
constexpr int kDropBatch = 8;

__device__ __forceinline__ float drop_wave_sum(float x) {
  x = group_sum<16>(x);
  x = sum_xor16(x);
  return sum_xor32(x);
}
__device__ __forceinline__ float drop_wave_max(float x) {
  x = group_max<16>(x);
  x = max_xor16(x);
  return max_xor32(x);
}

template <int V>  // tokens per load: 4 (aligned rows) or 1
__global__ __launch_bounds__(kDropThreads) void dropped_mass_kernel(DropArgs a) {
  constexpr int NT = kDropThreads, NW = NT / 64;
  __shared__ uint32_t s_kept[kMaxDropSeq / 32];
  __shared__ float s_r[3][NW];
  const Dims& d = a.d;
  const GroupBlock gb = group_block(d.B * d.Hkv);
  const int g = gb.bg % d.Hkv, b = gb.bg / d.Hkv, h = g * d.G + gb.j;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = clamp_len(a.seq_lens[b], d.max_seq);
  const int words = (n + 31) / 32;
  for (int w = tid; w < words; w += NT) s_kept[w] = 0u;
  __syncthreads();
  {
    const int32_t* list = a.sel_idx + (int64_t)gb.bg * a.k_max;
    const int cnt = max(0, min(a.sel_count[gb.bg], a.k_max));
    for (int e = tid; e < cnt; e += NT) {
      const int t = list[e];
      if (t >= 0 && t < n) atomicOr(&s_kept[t >> 5], 1u << (t & 31));
    }
  }
  __syncthreads();
  const float* row = a.logits + ((int64_t)b * d.Hq + h) * d.max_seq;
  const int32_t* bt = a.block_table + (int64_t)b * d.max_pages;
  // logits of tokens t .. t + V - 1 (t a multiple of V), -inf where not
  // attended; loads issued unconditionally with clamped indices (a branch
  // around them would drain each round)
  typedef float vec_t __attribute__((ext_vector_type(V)));
  auto logits_at = [&](int t) -> vec_t {
    const int tc = min(t, max(((n - 1) / V) * V, 0));
    const int ph = bt[min(tc / d.P, d.max_pages - 1)];
    const vec_t z = *reinterpret_cast<const vec_t*>(row + tc);
    const bool pg = (ph >= 0) & ((int64_t)ph < d.num_pages);
    vec_t out;
#pragma unroll
    for (int i = 0; i < V; ++i) out[i] = (pg & (t + i < n)) ? z[i] : -INFINITY;
    return out;
  };
  const int rounds = (n + NT * V - 1) / (NT * V);
  auto for_tokens = [&](auto&& fn) {
    for (int k0 = 0; k0 < rounds; k0 += kDropBatch) {
      vec_t zz[kDropBatch];
#pragma unroll
      for (int r = 0; r < kDropBatch; ++r) zz[r] = logits_at(((k0 + r) * NT + tid) * V);
#pragma unroll
      for (int r = 0; r < kDropBatch; ++r)
#pragma unroll
        for (int i = 0; i < V; ++i) fn(((k0 + r) * NT + tid) * V + i, zz[r][i]);
    }
  };
  float m = -INFINITY;
  for_tokens([&](int, float z) { m = fmaxf(m, z); });
  m = drop_wave_max(m);
  if (lane == 0) s_r[0][wave] = m;
  __syncthreads();
  m = -INFINITY;
#pragma unroll
  for (int w = 0; w < NW; ++w) m = fmaxf(m, s_r[0][w]);
  float* out = a.delta + (int64_t)b * d.Hq + h;
  if (m == -INFINITY) {  // no attended token: nothing to drop
    if (tid == 0) *out = 0.f;
    return;
  }
  float z_all = 0.f, z_drop = 0.f;
  for_tokens([&](int t, float z) {
    const float e = z == -INFINITY ? 0.f : expf(z - m);
    z_all += e;
    const bool kept = t < n && ((s_kept[min(t, n - 1) >> 5] >> (t & 31)) & 1u);
    z_drop += kept ? 0.f : e;
  });
  z_all = drop_wave_sum(z_all);
  z_drop = drop_wave_sum(z_drop);
  if (lane == 0) { s_r[1][wave] = z_all; s_r[2][wave] = z_drop; }
  __syncthreads();
  if (tid == 0) {
    float za = 0.f, zd = 0.f;
    for (int w = 0; w < NW; ++w) { za += s_r[1][w]; zd += s_r[2][w]; }
    *out = zd / za;
  }
}

hipError_t launch_dropped_mass(const DropArgs& a, hipStream_t st) {
  const Dims& d = a.d;
  if (d.max_seq > kMaxDropSeq || a.k_max < 1) return hipErrorInvalidValue;
  if ((d.max_seq & 3) == 0)
    dropped_mass_kernel<4><<<dim3(d.B * d.Hq), kDropThreads, 0, st>>>(a);
  else
    dropped_mass_kernel<1><<<dim3(d.B * d.Hq), kDropThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace sdkv
