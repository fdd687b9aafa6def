// Stage 1b: exact top-k of the unit scores of one (sequence, KV head).
//
// Keeps the k largest scores, equal scores going to the lower unit id, and
// writes the kept ids in ascending order (the selected block set over which
// attention runs: "SparDA: Sparse Decoupled Attention ..." summary, Section
// 3.1 and Appendix A).  k is the keep count of the sequence's U units in
// integer parts per million.
//
// Method: a float maps to an order-preserving 32-bit key (-0 folded onto +0);
// four 8-bit radix passes with an LDS histogram find the exact k-th largest
// key T and how many keys equal to T are still needed; a block-wide scan in
// index order then places every kept id.  All counting is integer, so the
// result does not depend on thread timing.
#include "device.h"

namespace sdkv {

constexpr int kSelectThreads = 1024;

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__global__ __launch_bounds__(kSelectThreads) void select_topk_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ seq_lens,
    int32_t* __restrict__ sel_idx, int32_t* __restrict__ sel_count, Dims d, int unit,
    int U_max, int k_max, int R_ppm) {
  constexpr int NW = kSelectThreads / 64;
  const int g = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = clamp_len(seq_lens[b], d.max_seq);
  int U = unit == kPage ? (n + d.P - 1) / d.P : n;
  U = min(U, U_max);
  int k;
  if (U == 0) {
    k = 0;
  } else if (R_ppm < 0) {
    k = U;
  } else {
    const int64_t kk = ((int64_t)R_ppm * U + 999999) / 1000000;
    k = (int)(kk < 1 ? 1 : (kk > U ? U : kk));
  }
  k = min(k, k_max);
  const int64_t bg = (int64_t)b * d.Hkv + g;
  const float* sc = scores + bg * U_max;
  int32_t* out = sel_idx + bg * k_max;
  if (tid == 0) sel_count[bg] = k;
  if (k == 0) return;
  if (k == U) {
    for (int i = tid; i < U; i += kSelectThreads) out[i] = i;
    return;
  }

  __shared__ uint32_t hist[256];
  __shared__ uint32_t s_prefix, s_need;
  __shared__ uint64_t s_wave[NW];

  uint32_t prefix = 0u, mask = 0u, need = (uint32_t)k;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    if (tid < 256) hist[tid] = 0u;
    __syncthreads();
    for (int i = tid; i < U; i += kSelectThreads) {
      const uint32_t key = order_key(sc[i]);
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      // lane j holds bins 255-4j .. 252-4j, so lanes run from the top bin down
      uint32_t c[4], tot = 0u;
#pragma unroll
      for (int i = 0; i < 4; ++i) { c[i] = hist[255 - 4 * lane - i]; tot += c[i]; }
      uint32_t run = wave_incl_scan(tot) - tot;  // keys in higher bins
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (run < need && run + c[i] >= need) {
          s_prefix = prefix | (uint32_t(255 - 4 * lane - i) << shift);
          s_need = need - run;
        }
        run += c[i];
      }
    }
    __syncthreads();
    prefix = s_prefix;
    need = s_need;
    mask |= 0xFFu << shift;
  }
  const uint32_t T = prefix;  // the k-th largest key; `need` keys equal to T are kept

  // Contiguous index range per thread, counted, scanned, then written in order.
  const int C = (U + kSelectThreads - 1) / kSelectThreads;
  const int lo = min(U, tid * C), hi = min(U, lo + C);
  uint32_t gt = 0u, eq = 0u;
  for (int i = lo; i < hi; ++i) {
    const uint32_t key = order_key(sc[i]);
    gt += key > T;
    eq += key == T;
  }
  const uint64_t v = (uint64_t(gt) << 32) | eq;
  const uint64_t incl = wave_incl_scan(v);
  if (lane == 63) s_wave[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    const uint64_t w = lane < NW ? s_wave[lane] : 0ull;
    const uint64_t wi = wave_incl_scan(w);
    if (lane < NW) s_wave[lane] = wi - w;
  }
  __syncthreads();
  const uint64_t excl = incl - v + s_wave[wave];
  const uint32_t gt_before = uint32_t(excl >> 32), eq_before = uint32_t(excl);
  uint32_t pos = gt_before + min(eq_before, need);
  uint32_t tie = eq_before;
  for (int i = lo; i < hi; ++i) {
    const uint32_t key = order_key(sc[i]);
    if (key > T) {
      if (pos < (uint32_t)k) out[pos] = i;
      ++pos;
    } else if (key == T) {
      if (tie < need) {
        if (pos < (uint32_t)k) out[pos] = i;
        ++pos;
      }
      ++tie;
    }
  }
}

hipError_t launch_select(const SelectArgs& a, hipStream_t st) {
  const dim3 grid(a.d.Hkv, a.d.B);
  select_topk_kernel<<<grid, kSelectThreads, 0, st>>>(a.unit_scores, a.seq_lens, a.sel_idx,
                                                      a.sel_count, a.d, a.unit, a.U_max,
                                                      a.k_max, a.R_ppm);
  return hipGetLastError();
}

}  // namespace sdkv
