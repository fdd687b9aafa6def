/*
 * sd.h -- C ABI of the MI355X (gfx950) sparse decode-attention library
 * (libsdkv.so).
 *
 * One decode step of grouped-query attention for B sequences, each with ONE
 * query token, over a paged KV cache, in two stages:
 *
 *   1. query-aware selection: every KV unit (a token, or a page of P tokens)
 *      is scored against the query -- by the exact logits q.K, or by a bound
 *      computed from per-page key minima and maxima -- and the top r_KV of
 *      the units are kept per (sequence, KV head);
 *   2. split-K attention over the kept units only: each split runs an online
 *      softmax over its share of the kept tokens, and the splits are merged
 *      by log-sum-exp.  Dense decoding is the same attention kernel with
 *      every unit kept.
 *
 * Sources (page title, then the part of the page):
 *   [Cross/cards] "Where Activation Sparsity and KV-Cache Sparsity Cross in
 *     LLM Decoding", cards view, EntmaxKV abstract: pages are scored against
 *     the query from light per-page statistics before they are loaded, then
 *     candidates are selected and attention runs on them; pre-hoc sparsity
 *     abstract: the dropped mass delta governs the error.
 *   [Cross/list] same title, list view, Abstract: attention-scored KV
 *     selection; dense and sparse decoding read the cache through one
 *     split-K attention kernel.  Tables 4 and 16: a keep ratio of 1 turns
 *     selection off.
 *   [SparDA] "SparDA: Sparse Decoupled Attention for Efficient Long-Context
 *     LLM Inference" summary page, Section 3.1: attention is computed over
 *     the attended blocks only; the query heads of a GQA group share one KV
 *     head and one block choice; initial, local and top-k blocks.
 *     Appendix A: the selected set as a union.  Appendix C: 64-token blocks.
 *
 * Conventions for every entry point
 *   - Pointers named *_host or the shape struct are host memory; every other
 *     pointer is device memory on the current HIP device.
 *   - The caller owns all buffers.  The library never allocates or frees
 *     memory; scratch space comes from the caller's workspace (ws, ws_bytes,
 *     256-byte aligned, contents need not be initialised).  Calls that share
 *     a workspace must not overlap in time (enqueue them on one stream).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     and runs asynchronously; nothing synchronises the host.
 *   - Host-visible arguments are validated before anything is enqueued.  On
 *     a non-OK status nothing has been enqueued or written, and
 *     sd_last_error() describes the failure (thread-local text).
 *   - Device-resident metadata is trusted only as far as memory safety goes:
 *     seq_lens[b] is clamped to [0, max_seq_len]; a block-table entry outside
 *     [0, num_pages) makes the kernels skip that page.  A sequence with no
 *     valid token yields out = 0 and lse = -inf.
 *
 * Layouts (row-major, innermost last)
 *   q            [B][H_q][d]              dtype
 *   k_pages      [num_pages][H_kv][P][d]  dtype  (one contiguous tile per
 *   v_pages      [num_pages][H_kv][P][d]  dtype   page and KV head)
 *   page_bounds  [B][H_kv][max_pages_per_seq][2][d]  dtype  per sequence, in
 *                logical page order (row 0: channel minima, row 1: maxima);
 *                entries past a sequence's last page are not read
 *   block_table  [B][max_pages_per_seq]   int32  physical page of logical page u
 *   seq_lens     [B]                      int32  valid tokens n_b
 *   unit_scores  [B][H_kv][U_max]         fp32   U_max = max_pages_per_seq
 *                                                 (page unit) or max_seq_len
 *                                                 (token unit)
 *   token_logits [B][H_q][max_seq_len]    fp32   (token unit only)
 *   sel_idx      [B][H_kv][k_max]         int32  kept unit ids, ascending
 *   sel_count    [B][H_kv]                int32  k_b per sequence
 *   out          [B][H_q][d]              fp32
 *   lse          [B][H_q]                 fp32   natural-log sum of exp(logits)
 * Query head h reads KV head h / G, G = H_q / H_kv.  Logical token t of
 * sequence b lives in page block_table[b][t / P], row t % P.
 */
#ifndef SPARSE_KV_SD_H
#define SPARSE_KV_SD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SD_API __attribute__((visibility("default")))

typedef enum sd_status {
  SD_OK = 0,
  SD_E_NULL = 1,         /* a required pointer is NULL */
  SD_E_SHAPE = 2,        /* inconsistent sizes */
  SD_E_DTYPE = 3,        /* unknown dtype */
  SD_E_RATIO = 4,        /* r_KV not finite or <= 0 */
  SD_E_WORKSPACE = 5,    /* ws too small or misaligned */
  SD_E_UNSUPPORTED = 6,  /* valid, but not built: d, P or G outside the supported set */
  SD_E_DEVICE = 7        /* the HIP runtime reported an error while enqueueing */
} sd_status;

typedef enum sd_dtype { SD_F32 = 0, SD_BF16 = 1 } sd_dtype;  /* q, K, V and page bounds */
typedef enum sd_unit { SD_UNIT_TOKEN = 0, SD_UNIT_PAGE = 1 } sd_unit;

/* Problem sizes (host struct). Supported: head_dim in {64, 128};
 * page_size in {16, 64}; G = num_q_heads / num_kv_heads in {1, 2, 4, 8}. */
typedef struct sd_shape {
  int32_t batch;              /* B >= 1 sequences, one query token each */
  int32_t num_q_heads;        /* H_q, a multiple of num_kv_heads */
  int32_t num_kv_heads;       /* H_kv >= 1 */
  int32_t head_dim;           /* d */
  int32_t page_size;          /* P tokens per page */
  int32_t max_pages_per_seq;  /* row length of block_table */
  int32_t max_seq_len;        /* >= every seq_lens[b]; <= max_pages_per_seq * P */
  int32_t dtype;              /* sd_dtype */
  int64_t num_pages;          /* physical pages in k_pages / v_pages / page_bounds */
  float softmax_scale;        /* multiplies q.K; <= 0 selects 1 / sqrt(d) */
} sd_shape;

/* Keep count for U units at keep ratio r_KV (host, pure): r_KV >= 1 keeps all
 * U; otherwise R = floor(r_KV * 1e6 + 0.5) parts per million and
 * k = ceil(R * U / 1e6) in integer arithmetic, clamped to [1, U].  The
 * kernels apply the same rule per sequence to U_b.  Returns -1 when r_KV is
 * not finite or <= 0, or U < 1. */
SD_API int32_t sd_keep_count(double r_kv, int32_t num_units);

/* Workspace bytes that suffice for every call below made with this shape,
 * unit and r_KV (sd_decode_step included), on the current device: the split
 * plan follows its compute-unit count (on a host with no GPU, 256, an
 * MI355X's).  Host only; enqueues nothing. */
SD_API sd_status sd_workspace_bytes(const sd_shape* shape, int32_t unit, double r_kv, size_t* bytes_host);

/* Setup step, not part of the decode step: the channel-wise min and max of
 * the keys of logical page u of sequence b (physical page
 * block_table[b][u]) over the page's VALID tokens only, written to
 * page_bounds[b][g][u] for every KV head g.  These are the light per-page
 * statistics of [Cross/cards] (EntmaxKV abstract), known before any page is
 * loaded.  Kept in logical order so that scoring needs no block-table lookup.
 *   pages == NULL: every page u < ceil(n_b / P) of every sequence.
 *   pages != NULL: only the n_pages listed (sequence, logical page) pairs
 *     (device int32 [n_pages][2]); pairs outside the batch or past a
 *     sequence's last page are skipped; n_pages = 0 enqueues nothing;
 *     SD_E_SHAPE if n_pages < 0.  A decode loop passes the pages its new
 *     tokens landed in.
 * A page whose block-table entry is outside [0, num_pages) is left as is. */
SD_API sd_status sd_update_page_bounds(const sd_shape* shape, const void* k_pages,
                                const int32_t* block_table, const int32_t* seq_lens,
                                const int32_t* pages, int32_t n_pages, void* page_bounds,
                                void* stream);

/* The per-token form of sd_update_page_bounds, O(d) per appended token and
 * KV head: sequence b gained the tokens n_b - a_b .. n_b - 1 since its
 * bounds were last current (seq_lens already counts them; a_b =
 * appended[b], device int32 [B], clamped to [0, min(n_b, max_appended)]).
 * Each such token is folded into its page's bounds (min with the stored
 * minima, max with the stored maxima); a page that an appended token opens
 * (its row 0 is appended) starts from that token.  The result equals a full
 * sd_update_page_bounds bit for bit, provided the bounds of the rows before
 * the first appended one were current.  max_appended (host) bounds every
 * a_b: SD_E_SHAPE outside [1, max_seq_len]. */
SD_API sd_status sd_append_page_bounds(const sd_shape* shape, const void* k_pages,
                                       const int32_t* block_table, const int32_t* seq_lens,
                                       const int32_t* appended, int32_t max_appended,
                                       void* page_bounds, void* stream);

/* Stage 1a, scoring ([Cross/cards] EntmaxKV abstract; [Cross/list] Abstract).
 *   unit == SD_UNIT_PAGE: reads q and page_bounds;
 *     unit_scores[b][g][u] = max over the G heads h of group g of
 *       scale * sum_c max(q[b][h][c] * kmin[c], q[b][h][c] * kmax[c]),
 *     an upper bound on every logit of page u; u < ceil(n_b / P).
 *     token_logits is not used (may be NULL).
 *   unit == SD_UNIT_TOKEN: reads q and every valid key;
 *     token_logits[b][h][t] = scale * q[b][h] . K[b][h / G][t] and
 *     unit_scores[b][g][t] = max over h in group g, for t < n_b.
 * Entries past a sequence's units are left untouched. */
SD_API sd_status sd_score_pages(const sd_shape* shape, const void* q, const void* k_pages,
                         const void* page_bounds, const int32_t* block_table,
                         const int32_t* seq_lens, int32_t unit, float* unit_scores,
                         float* token_logits, void* stream);

/* Stage 1b, exact top-k per (sequence b, KV head g): k_b = keep count of
 * U_b units; keeps the k_b largest unit_scores[b][g][0 .. U_b - 1], equal
 * scores going to the lower unit id (-0.0 equals +0.0), and writes them in
 * ascending order to sel_idx[b][g][0 .. k_b - 1]; sel_count[b][g] = k_b.
 * Scores must be finite.  k_max = sd_keep_count(r_kv, U_max) is the row
 * length of sel_idx.  Up to 16384 units per sequence one block selects each
 * (b, g) and ws may be NULL; beyond that the selection is spread over many
 * blocks per (b, g), whose scratch lives in ws (sd_workspace_bytes for this
 * shape and unit suffices; contents need not be set; SD_E_NULL /
 * SD_E_WORKSPACE when it is missing or too small). */
SD_API sd_status sd_select_topk(const sd_shape* shape, int32_t unit, const int32_t* seq_lens,
                         const float* unit_scores, double r_kv, int32_t* sel_idx,
                         int32_t* sel_count, void* ws, size_t ws_bytes, void* stream);

/* Stage 2, split-K attention over the kept units ([Cross/list] Abstract;
 * [SparDA] Section 3.1).  For each (b, g) the kept units
 * sel_idx[b][g][0 .. sel_count[b][g] - 1] are cut into splits; each split
 * keeps a running max, sum and weighted value sum over its tokens; splits are
 * merged by log-sum-exp into out[b][h] and lse[b][h].
 *   sel_idx == NULL: dense -- every unit of every sequence (sel_count unused).
 *   unit == SD_UNIT_PAGE: a kept page contributes its valid tokens.
 *   unit == SD_UNIT_TOKEN: sel_idx holds token ids; with token_logits != NULL
 *     the logits are read from there (written by sd_score_pages) and only V
 *     rows of the kept tokens are read; with NULL, q.K is recomputed.
 * k_max: row length of sel_idx (ignored when sel_idx == NULL). */
SD_API sd_status sd_attend_splitk(const sd_shape* shape, const void* q, const void* k_pages,
                           const void* v_pages, const int32_t* block_table,
                           const int32_t* seq_lens, int32_t unit, const int32_t* sel_idx,
                           const int32_t* sel_count, int32_t k_max, const float* token_logits,
                           float* out, float* lse, void* ws, size_t ws_bytes, void* stream);

/* Stage 2a alone: the split partials of the split-K attention, written to the
 * workspace (per split j of (b, g): the normalised output and log-sum-exp of
 * each head over the split's tokens).  The kept list comes from exactly one
 * source:
 *   sel_idx != NULL   the list ([B][H_kv][k_max], counts in sel_count);
 *   unit_scores != NULL  (page unit, bf16, <= 16384 pages per sequence) every
 *                     block runs the exact top-k of sd_select_topk on the page
 *                     scores itself and attends its share of the kept pages;
 *                     sel_out / sel_count_out, if given, receive the selection;
 *                     SD_E_UNSUPPORTED outside that range;
 *   neither           every unit (dense).
 * token_logits as in sd_attend_splitk.  Follow with sd_merge_splits on the
 * same workspace. */
SD_API sd_status sd_attend_partials(const sd_shape* shape, const void* q, const void* k_pages,
                             const void* v_pages, const int32_t* block_table,
                             const int32_t* seq_lens, int32_t unit, const int32_t* sel_idx,
                             const int32_t* sel_count, int32_t k_max, const float* token_logits,
                             const float* unit_scores, double r_kv, int32_t* sel_out,
                             int32_t* sel_count_out, void* ws, size_t ws_bytes, void* stream);

/* Stage 2b alone: log-sum-exp merge of the partials that the last
 * sd_attend_partials call on this workspace wrote (the split count is kept
 * in the workspace):  M = max_j lse_j, w_j = exp(lse_j - M),
 * out = sum_j w_j o_j / sum_j w_j, lse = M + log sum_j w_j. */
SD_API sd_status sd_merge_splits(const sd_shape* shape, float* out, float* lse, void* ws,
                          size_t ws_bytes, void* stream);

/* Stages 1b and 2 together, page unit: from the page scores of
 * sd_score_pages, the exact top-k (as sd_select_topk) and split-K attention
 * over the kept pages (as sd_attend_splitk).  For bf16 data with at most
 * 16384 pages per sequence, every attention block selects the pages of its
 * (sequence, KV head) itself and attends its share of them (one kernel, then
 * the merge); otherwise it runs top-k, attention and merge in turn.
 * sel_idx / sel_count may be NULL; when given they receive the selection
 * ([B][H_kv][k_max], [B][H_kv]).  ws as for sd_decode_step with page unit. */
SD_API sd_status sd_select_attend(const sd_shape* shape, const void* q, const void* k_pages,
                           const void* v_pages, const int32_t* block_table,
                           const int32_t* seq_lens, const float* unit_scores, double r_kv,
                           float* out, float* lse, int32_t* sel_idx, int32_t* sel_count,
                           void* ws, size_t ws_bytes, void* stream);

/* The whole decode step: r_kv >= 1 runs dense attention only; otherwise
 * scoring (by unit), top-k and attention over the kept units.  page_bounds
 * is read in page unit (built beforehand by sd_update_page_bounds).
 * sel_idx / sel_count may be NULL (then they live in ws); when given they
 * receive the selection ([B][H_kv][k_max], [B][H_kv]). */
SD_API sd_status sd_decode_step(const sd_shape* shape, const void* q, const void* k_pages,
                         const void* v_pages, const void* page_bounds,
                         const int32_t* block_table, const int32_t* seq_lens, int32_t unit,
                         double r_kv, float* out, float* lse, int32_t* sel_idx,
                         int32_t* sel_count, void* ws, size_t ws_bytes, void* stream);

/* ---- Structured index sets ----------------------------------------------
 * Which units a decode step keeps (host struct):
 *   SD_SEL_TOPK             the exact top-k of sd_select_topk, k_b = keep
 *                           count of U_b at r_kv;
 *   SD_SEL_WINDOW           the k_b most recent units U_b - k_b .. U_b - 1:
 *                           the KV-window baseline of [Cross/list] Table 3
 *                           (scores are not used);
 *   SD_SEL_INIT_LOCAL_TOPK  the union of the first init_units units, the last
 *                           local_units units and the top-k of all U_b units
 *                           ([SparDA] Section 3.1: initial, local and top-k
 *                           blocks; Appendix A: B_init U B_local U top-k);
 *   SD_SEL_MASS_BUDGET      token unit only: the shortest prefix of the top-k
 *                           order (decreasing score, equal scores to the lower
 *                           id) that leaves at most max_dropped of every
 *                           head's dense softmax mass outside, capped at k_b
 *                           ([Cross/cards] pre-hoc sparsity abstract: the
 *                           dropped mass controlled in advance).  Needs the
 *                           token logits; any number of tokens (one block per
 *                           (b, g) up to 8192, many past that: the same rule,
 *                           with the fp32 softmax normalisers summed in another
 *                           order).  The masses are summed as 2^-40
 *                           fixed-point integers of the fp32 softmax weights;
 *                           when no unit needs keeping to meet the target,
 *                           one unit is kept.
 * Lists are ascending.  The row length of a kept list is
 * sd_selection_capacity(sel, U_max): k_max, or min(U_max, init_units +
 * local_units + k_max) for the union. */
typedef enum sd_selection_kind {
  SD_SEL_TOPK = 0,
  SD_SEL_WINDOW = 1,
  SD_SEL_INIT_LOCAL_TOPK = 2,
  SD_SEL_MASS_BUDGET = 3
} sd_selection_kind;

typedef enum sd_scorer {
  SD_SCORER_BOUNDS = 0,     /* page bounds (sd_update_page_bounds) */
  SD_SCORER_COMPRESSED = 1  /* compressed keys (sd_update_compressed_keys) */
} sd_scorer;

typedef struct sd_selection {
  int32_t kind;         /* sd_selection_kind */
  int32_t init_units;   /* >= 0; SD_SEL_INIT_LOCAL_TOPK only */
  int32_t local_units;  /* >= 0; SD_SEL_INIT_LOCAL_TOPK only */
  int32_t scorer;       /* sd_scorer, page unit (token unit scores q.K) */
  double r_kv;          /* keep ratio of the top-k (window; the budget's cap,
                           where >= 1 means no cap rather than dense) */
  double max_dropped;   /* in [0, 1]; SD_SEL_MASS_BUDGET only */
} sd_selection;

/* ---- Compressed-key page scoring --------------------------------------
 * A second page scorer ([SparDA] Section 3.1: a parameter-free selector
 * mean-pools the keys into overlapping compressed representations, sums the
 * per-head relevance over the GQA group and max-pools it to the block score;
 * Appendix C: kernel 32, stride 16).  Layout:
 *   compressed_keys  [B][H_kv][W][d] fp32, W = ceil(max_seq_len / 16): window
 *                    j is the mean of the valid keys 16 j .. 16 j + 31 (fewer
 *                    at the end of a sequence; pages whose block-table entry
 *                    is invalid are left out of the mean).
 * Setup (not part of the decode step): sd_update_compressed_keys writes the
 * windows j < ceil(n_b / 16) of every sequence from the K pool.
 * Scoring: unit_scores[b][g][u] = max over the windows j that start in page
 * u (j = u P / 16 .. (u + 1) P / 16 - 1, j < ceil(n_b / 16)) of
 * scale * sum over the G heads h of group g of q[b][h] . c_j, for
 * u < ceil(n_b / P); page unit, P = 16 or 64. */
SD_API sd_status sd_update_compressed_keys(const sd_shape* shape, const void* k_pages,
                                           const int32_t* block_table, const int32_t* seq_lens,
                                           float* compressed_keys, void* stream);
SD_API sd_status sd_score_compressed(const sd_shape* shape, const void* q,
                                     const float* compressed_keys, const int32_t* seq_lens,
                                     float* unit_scores, void* stream);

/* Row length of a kept list for at most num_units units (host, pure); -1 on
 * an invalid selection or num_units < 1. */
SD_API int32_t sd_selection_capacity(const sd_selection* sel, int32_t num_units);

/* Workspace bytes that suffice for sd_select_units and sd_decode_step_sel
 * with this shape, unit and selection (and for every call that
 * sd_workspace_bytes covers at sel->r_kv).  Host only. */
SD_API sd_status sd_workspace_bytes_sel(const sd_shape* shape, int32_t unit,
                                        const sd_selection* sel, size_t* bytes_host);

/* Stage 1b under a selection: writes the kept units of every (b, g),
 * ascending, to sel_idx[b][g][0 .. sel_count[b][g] - 1] (rows of
 * sd_selection_capacity(sel, U_max) entries).  unit_scores as for
 * sd_select_topk (may be NULL for SD_SEL_WINDOW).  The union is the top-k of
 * sd_select_topk merged with the two ranges.  token_logits (as written by
 * sd_score_pages) is read by SD_SEL_MASS_BUDGET only and may be NULL
 * otherwise.  ws: sd_workspace_bytes_sel. */
SD_API sd_status sd_select_units(const sd_shape* shape, int32_t unit, const int32_t* seq_lens,
                                 const float* unit_scores, const float* token_logits,
                                 const sd_selection* sel, int32_t* sel_idx, int32_t* sel_count,
                                 void* ws, size_t ws_bytes, void* stream);

/* sd_decode_step under a selection.  SD_SEL_TOPK is sd_decode_step at
 * sel->r_kv.  SD_SEL_WINDOW attends the window directly (no scoring;
 * page_bounds not read).  SD_SEL_INIT_LOCAL_TOPK scores, selects the union
 * and attends it; in page unit with bf16 data and at most 16384 pages per
 * sequence the attention blocks select it themselves, as in
 * sd_select_attend.  With sel->scorer == SD_SCORER_COMPRESSED (page unit)
 * page_bounds must point to the compressed keys ([B][H_kv][W][d] fp32) and
 * the pages are scored by sd_score_compressed.  SD_SEL_MASS_BUDGET scores the
 * tokens, selects with the
 * budget and attends over the stored logits.  sel_idx / sel_count may be
 * NULL; when given they receive the kept lists (rows of
 * sd_selection_capacity(sel, U_max)).
 * ws: sd_workspace_bytes_sel. */
SD_API sd_status sd_decode_step_sel(const sd_shape* shape, const void* q, const void* k_pages,
                                    const void* v_pages, const void* page_bounds,
                                    const int32_t* block_table, const int32_t* seq_lens,
                                    int32_t unit, const sd_selection* sel, float* out,
                                    float* lse, int32_t* sel_idx, int32_t* sel_count, void* ws,
                                    size_t ws_bytes, void* stream);

/* ---- alpha-entmax attention over the kept set ---------------------------
 * [Cross/cards] EntmaxKV abstract: alpha-entmax attention gives exact zeros,
 * so sparse decoding becomes support recovery -- when the kept candidates
 * hold the entmax support the sparse output equals the dense one; otherwise
 * the error is governed by the dropped mass delta.  The scores, the kept
 * lists and the split-K structure are those of sd_decode_step_sel; only the
 * weights differ.  For query head h of sequence b over its kept tokens T:
 *   z_t = scale * q[b][h] . K_t,   x_t = (alpha - 1) z_t,
 *   p_t = max(x_t - tau, 0) ** (1 / (alpha - 1)),  sum_{t in T} p_t = 1,
 *   out[b][h] = sum_{t in T} p_t V_t,   tau[b][h] = tau.
 * alpha = 2 is sparsemax; 1.5 is the usual entmax; alpha -> 1 tends to
 * softmax.  The steps: scoring and selection as sd_decode_step_sel (the
 * same scorer, keep count, top-k, window, union or budget); the logits of
 * the kept tokens (token unit: those of the token scorer; page unit, a
 * window or every unit: a logits-only pass of the attention kernel over the
 * kept list, which reads K but not V; in page unit with the top-k or the
 * union this pass also selects the pages); tau per head by Newton steps,
 * in fp32, on (sum max(x - tau, 0)^(1/(alpha-1)))^(alpha-1) - 1 from
 * tau = max x - 1, which climb monotonically to the root (one block per
 * head, or past 16384 kept tokens a block per 16384 of them and a merge
 * block; at most 1024 such blocks, 16777216 kept tokens per head:
 * SD_E_UNSUPPORTED beyond); split-K attention with these weights over the stored logits
 * (reads V), merged as sum_j a_j / sum_j l_j, which also removes the
 * residual of tau's rounding.  Launches use the caller's workspace only.
 *   page_stats  as page_bounds of sd_decode_step_sel (the page bounds, or
 *               the compressed keys with sel->scorer == SD_SCORER_COMPRESSED);
 *               not read in token unit, for a window or with r_kv >= 1.
 *   alpha       in (1, 2]; SD_E_RATIO otherwise.
 *   out         [B][H_q][d] fp32.
 *   tau         [B][H_q] fp32 or NULL: the threshold of every head (+inf for
 *               a sequence with no attended token, whose out is 0).
 *   sel_idx / sel_count  as for sd_decode_step_sel (not written when every
 *               unit is kept).
 *   ws          sd_workspace_bytes_entmax bytes (contents need not be set).
 * The dropped-mass budget (SD_SEL_MASS_BUDGET) still measures softmax mass. */
SD_API sd_status sd_workspace_bytes_entmax(const sd_shape* shape, int32_t unit,
                                           const sd_selection* sel, size_t* bytes_host);
SD_API sd_status sd_decode_step_entmax(const sd_shape* shape, const void* q, const void* k_pages,
                                       const void* v_pages, const void* page_stats,
                                       const int32_t* block_table, const int32_t* seq_lens,
                                       int32_t unit, const sd_selection* sel, double alpha,
                                       float* out, float* tau, int32_t* sel_idx,
                                       int32_t* sel_count, void* ws, size_t ws_bytes,
                                       void* stream);

/* ---- Dropped mass on the device (token unit) -------------------------
 * [Cross/cards] pre-hoc sparsity abstract: the dropped mass delta -- the
 * dense attention probability of the entries a selection leaves out --
 * governs the error of sparse attention ([Cross/cards] EntmaxKV abstract:
 * ||o - o_S|| <= 2 delta max ||v||).  In token unit every logit is stored,
 * so delta costs one more pass over them:
 *   delta[b][h] = sum over the attended tokens t of sequence b NOT in
 *                 sel_idx[b][h / G][0 .. sel_count - 1] of exp(s_t - m)
 *                 / sum over all its attended tokens of exp(s_t - m),
 * s = token_logits[b][h] (as sd_score_pages writes them), m their max; a
 * token is attended when t < seq_lens[b] and its page's block-table entry
 * is valid.  The dropped tokens are summed directly (not as one minus the
 * kept mass), in fp32 and a fixed order; list entries outside [0, n_b) are
 * ignored; a sequence with no attended token gets delta = 0.
 *   sel_idx / sel_count: token ids as sd_select_topk or sd_select_units
 *   write them ([B][H_kv][k_max], [B][H_kv]); any ascending or unordered
 *   set of distinct ids works.
 *   delta: [B][H_q] fp32.
 * max_seq_len <= 262144 (SD_E_UNSUPPORTED beyond). */
SD_API sd_status sd_dropped_mass(const sd_shape* shape, const int32_t* seq_lens,
                                 const int32_t* block_table, const float* token_logits,
                                 const int32_t* sel_idx, const int32_t* sel_count, int32_t k_max,
                                 float* delta, void* stream);

/* ---- Allocation-free decode step -------------------------------------
 * For callers that cannot allocate device memory or pass a workspace: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  The same work as sd_decode_step (same arguments without ws /
 * ws_bytes, same kernels, same results), with its scratch space in a static
 * device array of 32 MiB that the library holds on every device it runs on
 * until the process ends.  The call allocates and frees nothing.
 *   - Shapes whose sd_workspace_bytes exceeds 32 MiB are refused with
 *     SD_E_WORKSPACE before anything is enqueued (every configuration of the
 *     benchmark fits; 1M-token token-unit steps do not).
 *   - Calls on one device share that device's array: calls that overlap in
 *     time on one device (different streams, or several host threads) race
 *     and give undefined results.  Enqueue them on one stream.  Nothing in
 *     the array needs clearing between calls: every region is written before
 *     it is read, as with a caller workspace.
 *   - The first call on a device looks up the array's device address
 *     (SD_E_DEVICE if that fails). */
SD_API sd_status sd_decode_step_noalloc(const sd_shape* shape, const void* q, const void* k_pages,
                                        const void* v_pages, const void* page_bounds,
                                        const int32_t* block_table, const int32_t* seq_lens,
                                        int32_t unit, double r_kv, float* out, float* lse,
                                        int32_t* sel_idx, int32_t* sel_count, void* stream);

/* Text of the last non-OK status on this thread ("" if none). */
SD_API const char* sd_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_KV_SD_H */
