// Internal interface between the C ABI (abi.cpp) and the HIP kernels.
// Not installed; the public interface is include/sd.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdkv {

enum Unit : int { kToken = 0, kPage = 1 };
enum DType : int { kF32 = 0, kBF16 = 1 };

// Problem sizes shared by every launch.
struct Dims {
  int B, Hq, Hkv, G, D, P;
  int max_pages, max_seq;
  int dtype;
  int64_t num_pages;
  float scale;  // softmax scale on q.K (natural-log domain)
};

struct BoundsArgs {
  Dims d;
  const void* k_pages;
  const int32_t* block_table;
  const int32_t* seq_lens;
  void* bounds;
  // At most one of the two: pages ([n_pages][2] (sequence, logical page)
  // pairs to recompute) or appended ([B] tokens that joined each sequence
  // since the bounds were last current, folded in; at most max_appended
  // each).  Neither: every page.
  const int32_t* pages = nullptr;
  int n_pages = 0;
  const int32_t* appended = nullptr;
  int max_appended = 0;
};

struct ScoreArgs {
  Dims d;
  int unit;
  const void* q;
  const void* k_pages;
  const void* bounds;
  const int32_t* block_table;
  const int32_t* seq_lens;
  float* unit_scores;   // [B][Hkv][U_max]
  float* token_logits;  // [B][Hq][max_seq] (token unit), or token-major (below)
  // Optional (token unit): per scoring block, the min and max order keys of
  // its valid unit scores, [B*Hkv][ceil(max_seq / score_units_per_block)][2].
  uint32_t* score_mm;
  // Token unit: logits_tm != 0 lays token_logits out token-major,
  // [B][Hkv][max_seq][G] (the G logits of a token adjacent), for readers
  // inside one decode step; 0 is the public [B][Hq][max_seq].
  int logits_tm = 0;
};

// Units one token-scoring block covers (the stride of ScoreArgs::score_mm).
int score_units_per_block(int dtype, int D);

struct SelectArgs {
  Dims d;
  int unit;
  const int32_t* seq_lens;
  const float* unit_scores;  // [B][Hkv][U_max]
  int U_max;
  int k_max;
  int R_ppm;  // keep ratio in parts per million; < 0 keeps every unit
  int32_t* sel_idx;    // [B][Hkv][k_max]
  int32_t* sel_count;  // [B][Hkv]
};

// Units per slice of the many-block top-k (select_multi.hip).
constexpr int kSliceUnits = 4096;

// Where the many-block top-k's first two launches (value histograms, then
// the bin of the k-th largest score and its candidates) leave their results,
// for a placement of the kept units that another kernel runs.
struct SliceSel {
  int NB = 0;                     // slices per (sequence, KV head); 0: none
  const float* scores = nullptr;  // [B][Hkv][U_max] unit scores
  const uint32_t* mm = nullptr;   // [B*Hkv][mm_nb][2] partial min / max keys
  int mm_nb = 0, mm_per = 0;
  const uint32_t* above = nullptr;   // [B*Hkv][NB] keys above the bin, per slice
  const uint32_t* ccount = nullptr;  // [B*Hkv][NB] keys in the bin, per slice
  const uint2* cand = nullptr;       // [B*Hkv][NB][64] (key, unit) candidates
};

struct AttendArgs {
  Dims d;
  int unit;
  const void* q;
  const void* k_pages;
  const void* v_pages;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* sel_idx;    // NULL: every unit
  const int32_t* sel_count;
  int k_max;
  const float* token_logits;  // token unit: read logits instead of q.K
  int logits_tm;              // token_logits token-major (ScoreArgs::logits_tm)
  int E;                      // kept units per split
  int S;                      // splits per (sequence, KV head), <= kMaxSplits
  float* part_o;              // [B][Hq][S][D]  split outputs, normalised
  float* part_lse;            // [B][Hq][S]     split log-sum-exp (-inf: empty)
  int32_t* split_count;       // S, written for the merge kernel
  // In-kernel selection (page unit, bf16): when unit_scores is set, every
  // block selects the top-k pages of its (sequence, KV head) itself and
  // attends its slice of them; sel_idx must then be NULL.
  const float* unit_scores;   // [B][Hkv][max_pages]
  int R_ppm;                  // keep ratio in parts per million (< 0: all)
  int32_t* sel_out;           // optional [B][Hkv][k_max]: kept list (split 0 writes it)
  int32_t* sel_count_out;     // optional [B][Hkv]
  // In-kernel selection: the first force_init and the last force_local units
  // are kept besides the top-k (their union, at most k_max units).
  int force_init, force_local;
  // Without a list or scores: window != 0 attends only the last
  // keep_count(U, R_ppm) units (list entry e is unit U - k + e).
  int window;
  // alpha-entmax weights instead of softmax (needs token_logits): token t of
  // head h weighs max(alpha_m1 * logit - tau[b][h], 0) ** beta with
  // alpha_m1 = alpha - 1 and beta = 1 / (alpha - 1); a split then reports
  // log(sum of its weights) as its lse.
  const float* tau;           // [B][Hq], NULL: softmax
  float alpha_m1, beta;
  // logits_out != NULL: no attention; the logits scale * q.K of every
  // attended token are written to logits_out [B][Hq][max_seq] (V not read).
  float* logits_out;
  // bf16 only: logits_out, and token_logits when read, are indexed by kept
  // slot instead of token: slot e * P + r for row r of the page at list
  // entry e (page unit), e for list entry e (token unit), so a split's slots
  // are one contiguous run.  The logits-only pass then also writes -inf to
  // the slots of its list range that it does not attend.
  int logits_slots;
  // Token unit, bf16, with sl.NB > 0: the kept list is placed inside the
  // kernel from the many-block top-k's candidates (sel_idx, unit_scores
  // NULL; softmax over token_logits, token-major).  Split j of (b, g) covers
  // units [j R, (j + 1) R), R = kSliceUnits >> sub_log2 (S = NB << sub_log2):
  // every block finds the kept units of its slice as the placement launch
  // would (keep count min(keep_count(U, R_ppm), k_max)), attends those in
  // its range and writes them to sel_out [B][Hkv][k_max] at their place in
  // the group's list (split 0 writes sel_count_out).
  SliceSel sl;
  int sub_log2;
};

// alpha-entmax threshold of every (sequence, query head) over the logits of
// the tokens of its kept list (or of every unit without a list), one block
// per head: tau with sum_t max(alpha_m1 * logit_t - tau, 0) ** beta = 1.
// Tokens on pages with an invalid block-table entry are left out, as the
// attention kernel leaves them out.
struct TauArgs {
  Dims d;
  int unit;
  const int32_t* seq_lens;
  const int32_t* block_table;
  const int32_t* sel_idx;    // NULL: every unit
  const int32_t* sel_count;
  int k_max;
  const float* logits;       // [B][Hq][max_seq]
  float alpha_m1, beta;
  float* tau;                // [B][Hq]
  // More than kTauChunk kept slots per head: nch chunks of kTauChunk slots,
  // one block each, leave their max and their candidates in cand / cmax /
  // ccnt ([B*Hq][nch][kTauChunkCap], [B*Hq][nch], [B*Hq][nch]); a second
  // kernel merges them.  nch = 0: one block per head does everything.
  int nch;
  float* cand;
  float* cmax;
  int32_t* ccnt;
  // logits indexed by kept slot (AttendArgs::logits_slots): slot i's logit is
  // logits[(b*Hq + h)*max_seq + i], -inf where nothing is attended; the list
  // and block table are then not read
  int logits_slots;
};
constexpr int kTauChunk = 16384;     // kept slots per threshold block
constexpr int kTauChunkCap = 2048;   // candidates a chunk hands on
constexpr int kTauMaxChunks = 1024;  // chunks per head (one per merge thread)
hipError_t launch_entmax_tau(const TauArgs& a, hipStream_t st);

// Dropped mass of the dense softmax (token unit), one block per (sequence,
// query head): delta[b][h] = sum over the attended tokens NOT in the kept
// list of (b, h / G) of exp(s_t - m) / sum over all attended tokens of
// exp(s_t - m), m the max logit.  A token is attended when t < n_b and its
// page's block-table entry is valid.  max_seq <= kMaxDropSeq (the kept set
// is a bitmap in LDS).
struct DropArgs {
  Dims d;
  const int32_t* seq_lens;
  const int32_t* block_table;
  const float* logits;       // [B][Hq][max_seq]
  const int32_t* sel_idx;    // [B][Hkv][k_max] token ids
  const int32_t* sel_count;  // [B][Hkv]
  int k_max;
  float* delta;              // [B][Hq]
};
constexpr int kMaxDropSeq = 262144;
hipError_t launch_dropped_mass(const DropArgs& a, hipStream_t st);

// Structured kept lists, one block per (sequence, KV head): kind kWindow
// writes the last keep_count(U, R_ppm) units; kind kInitLocalTopk writes the
// union of the first init_units, the last local_units and the ascending
// top-k list topk_idx (topk_count entries, row stride topk_stride), which
// must not alias sel_idx.  Rows of sel_idx hold cap entries.
enum StructKind : int { kWindow = 1, kInitLocalTopk = 2 };
struct StructArgs {
  Dims d;
  int unit;
  const int32_t* seq_lens;
  int kind;
  int R_ppm;
  int init_units, local_units;
  const int32_t* topk_idx;
  const int32_t* topk_count;
  int topk_stride;
  int32_t* sel_idx;    // [B][Hkv][cap]
  int32_t* sel_count;  // [B][Hkv]
  int cap;
};
hipError_t launch_structure(const StructArgs& a, hipStream_t st);

// Top-k with a dropped-mass budget (token unit), one block per (sequence, KV
// head), U_max <= kMaxSelectOne, G <= 8: the shortest prefix of the top-k
// order leaving at most max_dropped of every head's dense softmax mass
// outside, capped at min(keep_count(U, R_ppm), k_max).  logits: the token
// scorer's [B][Hq][max_seq].
struct BudgetArgs {
  Dims d;
  const int32_t* seq_lens;
  const float* scores;   // [B][Hkv][U_max]
  const float* logits;
  int U_max, k_max, R_ppm;
  float max_dropped;
  int32_t* sel_idx;      // [B][Hkv][k_max]
  int32_t* sel_count;    // [B][Hkv]
};
hipError_t launch_select_budget(const BudgetArgs& a, hipStream_t st);
// The same rule spread over many blocks per (b, g): any U_max
// (<= max_seq), G <= 8; scratch of budget_multi_workspace_bytes(d, U_max)
// bytes (contents need not be set).
size_t budget_multi_workspace_bytes(const Dims& d, int U_max);
hipError_t launch_select_budget_multi(const BudgetArgs& a, void* ws, hipStream_t st);

// Compressed-key page scoring.  ckeys: [B][Hkv][max_windows][D] fp32, window
// j the mean of the valid keys 16 j .. 16 j + 31 (max_windows =
// compressed_windows(d)).  launch_compress_keys writes ckeys from the K pool;
// launch_score_compressed writes unit_scores [B][Hkv][max_pages] (page unit,
// P = 16 or 64) from q and ckeys.
struct CompressArgs {
  Dims d;
  const void* k_pages;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const void* q;
  float* ckeys;
  int max_windows;
  float* unit_scores;
};
int compressed_windows(const Dims& d);
hipError_t launch_compress_keys(const CompressArgs& a, hipStream_t st);
hipError_t launch_score_compressed(const CompressArgs& a, hipStream_t st);

// Most splits one (sequence, KV head) is cut into.
constexpr int kMaxSplits = 256;
// Largest slice of the kept list a selecting attention block may own, and
// the most units it can select from.
constexpr int kMaxSelectE = 2048;
constexpr int kMaxSelectU = 16384;
// Most units the one-block selection kernel takes (more: select_multi.hip).
constexpr int kMaxSelectOne = 32768;
// Most units the library gives the one-block top-k; past this the many-block
// top-k runs (slices of 4096 units: measured faster at 32768 token units,
// 54.4 against 56.8 us per step).
constexpr int kOneBlockTopkMax = 16384;

hipError_t launch_page_bounds(const BoundsArgs& a, hipStream_t st);
hipError_t launch_score(const ScoreArgs& a, hipStream_t st);
// One block per (sequence, KV head); U_max <= kMaxSelectOne.
hipError_t launch_select(const SelectArgs& a, hipStream_t st);
// Many blocks per (sequence, KV head), any U_max; scratch of
// msel_workspace_bytes(B, Hkv, U_max) bytes (contents need not be set).
// mm: partial min / max keys of the scores ([B*Hkv][mm_nb][2], each over
// mm_per consecutive units, e.g. ScoreArgs::score_mm), or NULL to compute
// them here.  k_of: the count to keep per (b, g) ([B*Hkv], at most k_max),
// or NULL for min(keep_count(U, R_ppm), k_max).
size_t msel_workspace_bytes(int B, int Hkv, int U_max);
hipError_t launch_select_multi(const SelectArgs& a, const uint32_t* mm, int mm_nb, int mm_per,
                               void* ws, hipStream_t st, const int32_t* k_of = nullptr);
// The first two launches only (mm given, k_of NULL); *out receives where
// their results live, for the attention kernel's placement (AttendArgs::sl).
hipError_t launch_select_multi_bins(const SelectArgs& a, const uint32_t* mm, int mm_nb,
                                    int mm_per, void* ws, hipStream_t st, SliceSel* out);
// Log-sum-exp merge of the split partials written by an attention launch.
struct MergeArgs {
  Dims d;
  const float* part_o;
  const float* part_lse;
  const int32_t* split_count;
  int S_max;
  int S_known;                // > 0: the split count (no read of split_count)
  float* out;                 // [B][Hq][D]
  float* lse;                 // [B][Hq]
};

hipError_t launch_attend(const AttendArgs& a, hipStream_t st);
hipError_t launch_merge(const MergeArgs& a, hipStream_t st);

}  // namespace sdkv
