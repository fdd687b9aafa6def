// Stage 1b: exact top-k of the unit scores of one (sequence, KV head), as a
// standalone kernel: one block per (sequence, KV head).  The search itself
// (radix bins over the block's key range, ties to the lower index, ids in
// ascending order) is in topk.h.  The block's threads hold the keys in
// registers (up to 32768 units; more go to select_multi.hip, which spreads
// one selection over many blocks).
#include "topk.h"

namespace sdkv {

template <int NT, int KPT>
__global__ __launch_bounds__(NT) void select_topk_regs_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ seq_lens,
    int32_t* __restrict__ sel_idx, int32_t* __restrict__ sel_count, Dims d, int unit, int U_max,
    int k_max, int R_ppm) {
  __shared__ RadixState st;
  __shared__ KeptScratch<KPT, NT / 64> ks;
  const int g = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x;
  const int64_t bg = (int64_t)b * d.Hkv + g;
  const float* sc = scores + bg * U_max;
  // keys (interleaved: unit tid + NT*i) are read before the length is known
  uint32_t key[KPT];
#pragma unroll
  for (int i = 0; i < KPT; ++i) key[i] = order_key(sc[min(tid + NT * i, U_max - 1)]);
  const int n = clamp_len(seq_lens[b], d.max_seq);
  const int U = min(unit == kPage ? (n + d.P - 1) / d.P : n, U_max);
  const int k = min(keep_count_dev(U, R_ppm), k_max);
  int32_t* out = sel_idx + bg * k_max;
  if (tid == 0) sel_count[bg] = k;
  if (k == 0) return;
  if (k == U) {
    for (int i = tid; i < U; i += NT) out[i] = i;
    return;
  }
  topk_bitmap<KPT, NT / 64>(st, ks, key, U, k);
  emit_kept<KPT, NT / 64>(ks.mask, ks.base, 0u, (uint32_t)k,
                          [&](int pos, int unit_id) { out[pos] = unit_id; });
}

hipError_t launch_select(const SelectArgs& a, hipStream_t st) {
  const dim3 grid(a.d.Hkv, a.d.B);
  const int U = a.U_max;
#define SD_SELECT_REGS(NT, KPT)                                                              \
  select_topk_regs_kernel<NT, KPT><<<grid, NT, 0, st>>>(a.unit_scores, a.seq_lens, a.sel_idx, \
                                                        a.sel_count, a.d, a.unit, a.U_max,    \
                                                        a.k_max, a.R_ppm)
  if (U <= 2048) SD_SELECT_REGS(512, 4);
  else if (U <= 4096) SD_SELECT_REGS(512, 8);
  else if (U <= 8192) SD_SELECT_REGS(512, 16);
  else if (U <= 16384) SD_SELECT_REGS(1024, 16);
  else if (U <= kMaxSelectOne) SD_SELECT_REGS(1024, 32);
  else return hipErrorInvalidValue;  // many units: launch_select_multi
#undef SD_SELECT_REGS
  return hipGetLastError();
}

}  // namespace sdkv
