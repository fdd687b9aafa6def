// C ABI of libsdkv.so (declared in include/sd.h): argument validation, the
// split plan, workspace carving and kernel launches.  Host code only.
#include "sd.h"

#include <hip/hip_runtime_api.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "kernels.h"

namespace {

thread_local char g_err[512] = "";

sd_status fail(sd_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

sd_status ok() {
  g_err[0] = '\0';
  return SD_OK;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Attention blocks the split plan aims for: one 8-wave block per compute unit
// of the current device (asked once per device; 256 on an MI355X), or
// SD_ATTEND_BLOCKS when set (read once).  Without a device (sizing a
// workspace on a host with no GPU) the MI355X's 256 is assumed; a call on a
// device with more compute units then finds that workspace too small and
// says so (SD_E_WORKSPACE), as the plan is recomputed at every call.
constexpr int kMaxDevices = 64;
constexpr int64_t kDefaultBlocks = 256;

int64_t target_blocks() {
  static const int64_t env = [] {
    const char* e = std::getenv("SD_ATTEND_BLOCKS");
    const long x = e ? std::strtol(e, nullptr, 10) : 0;
    return static_cast<int64_t>(x > 0 ? x : 0);
  }();
  if (env > 0) return env;
  static std::atomic<int> cus[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return kDefaultBlocks;
  }
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n < 1) {
      (void)hipGetLastError();
      return kDefaultBlocks;
    }
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Parts-per-million keep ratio; -1 keeps everything (r >= 1).
int ratio_ppm(double r) {
  if (r >= 1.0) return -1;
  return static_cast<int>(std::floor(r * 1e6 + 0.5));
}

int64_t keep_count_ppm(int R, int64_t U) {
  if (U < 1) return 0;
  if (R < 0) return U;
  int64_t k = ceil_div(static_cast<int64_t>(R) * U, 1000000);
  return k < 1 ? 1 : (k > U ? U : k);
}

sd_status check_shape(const sd_shape* s, sdkv::Dims* d) {
  if (!s) return fail(SD_E_NULL, "shape is NULL");
  if (s->batch < 1 || s->num_q_heads < 1 || s->num_kv_heads < 1 || s->head_dim < 1 ||
      s->page_size < 1 || s->max_pages_per_seq < 1 || s->max_seq_len < 1 || s->num_pages < 1)
    return fail(SD_E_SHAPE, "every size in the shape must be >= 1");
  if (s->num_q_heads % s->num_kv_heads != 0)
    return fail(SD_E_SHAPE, "num_q_heads (%d) is not a multiple of num_kv_heads (%d)",
                s->num_q_heads, s->num_kv_heads);
  if (static_cast<int64_t>(s->max_seq_len) >
      static_cast<int64_t>(s->max_pages_per_seq) * s->page_size)
    return fail(SD_E_SHAPE, "max_seq_len (%d) exceeds max_pages_per_seq * page_size",
                s->max_seq_len);
  if (s->dtype != SD_F32 && s->dtype != SD_BF16)
    return fail(SD_E_DTYPE, "dtype %d is neither SD_F32 nor SD_BF16", s->dtype);
  const int G = s->num_q_heads / s->num_kv_heads;
  if (s->head_dim != 64 && s->head_dim != 128)
    return fail(SD_E_UNSUPPORTED, "head_dim %d not built (64 or 128)", s->head_dim);
  if (s->page_size != 16 && s->page_size != 64)
    return fail(SD_E_UNSUPPORTED, "page_size %d not built (16 or 64)", s->page_size);
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(SD_E_UNSUPPORTED, "group size %d not built (1, 2, 4 or 8)", G);
  if (!std::isfinite(s->softmax_scale))
    return fail(SD_E_SHAPE, "softmax_scale is not finite");
  d->B = s->batch;
  d->Hq = s->num_q_heads;
  d->Hkv = s->num_kv_heads;
  d->G = G;
  d->D = s->head_dim;
  d->P = s->page_size;
  d->max_pages = s->max_pages_per_seq;
  d->max_seq = s->max_seq_len;
  d->dtype = s->dtype;
  d->num_pages = s->num_pages;
  d->scale = s->softmax_scale > 0.f ? s->softmax_scale
                                    : 1.0f / std::sqrt(static_cast<float>(s->head_dim));
  return SD_OK;
}

sd_status check_unit(int unit) {
  if (unit != SD_UNIT_TOKEN && unit != SD_UNIT_PAGE)
    return fail(SD_E_SHAPE, "unit %d is neither SD_UNIT_TOKEN nor SD_UNIT_PAGE", unit);
  return SD_OK;
}

sd_status check_ratio(double r) {
  if (!std::isfinite(r) || r <= 0.0) return fail(SD_E_RATIO, "r_kv must be finite and > 0");
  return SD_OK;
}

int units_max(const sdkv::Dims& d, int unit) {
  return unit == SD_UNIT_PAGE ? d.max_pages : d.max_seq;
}

// A validated selection (include/sd.h, structured index sets).
struct Sel {
  int kind;  // SD_SEL_*
  double r;
  int init, local;  // SD_SEL_INIT_LOCAL_TOPK only (else 0)
  double dmax;      // SD_SEL_MASS_BUDGET only
  int scorer = SD_SCORER_BOUNDS;
};

Sel topk_sel(double r) { return Sel{SD_SEL_TOPK, r, 0, 0, 0.0, SD_SCORER_BOUNDS}; }

sd_status check_selection(const sd_selection* s, Sel* out) {
  if (!s) return fail(SD_E_NULL, "sel is NULL");
  if (s->kind != SD_SEL_TOPK && s->kind != SD_SEL_WINDOW && s->kind != SD_SEL_INIT_LOCAL_TOPK &&
      s->kind != SD_SEL_MASS_BUDGET)
    return fail(SD_E_SHAPE, "unknown selection kind %d", s->kind);
  if (s->kind == SD_SEL_MASS_BUDGET &&
      !(std::isfinite(s->max_dropped) && s->max_dropped >= 0.0 && s->max_dropped <= 1.0))
    return fail(SD_E_RATIO, "max_dropped must be in [0, 1]");
  sd_status st;
  if ((st = check_ratio(s->r_kv)) != SD_OK) return st;
  if (s->init_units < 0 || s->local_units < 0)
    return fail(SD_E_SHAPE, "init_units and local_units must be >= 0");
  const bool u = s->kind == SD_SEL_INIT_LOCAL_TOPK;
  if (s->scorer != SD_SCORER_BOUNDS && s->scorer != SD_SCORER_COMPRESSED)
    return fail(SD_E_SHAPE, "unknown scorer %d", s->scorer);
  *out = Sel{s->kind, s->r_kv, u ? s->init_units : 0, u ? s->local_units : 0,
              s->kind == SD_SEL_MASS_BUDGET ? s->max_dropped : 0.0, s->scorer};
  return SD_OK;
}

// The dropped-mass budget's limits: token unit.
sd_status check_budget(const sdkv::Dims& d, int unit, const Sel& s) {
  (void)d;
  if (s.kind != SD_SEL_MASS_BUDGET) return SD_OK;
  if (unit != SD_UNIT_TOKEN)
    return fail(SD_E_UNSUPPORTED, "the dropped-mass budget is token unit only");
  return SD_OK;
}

// Row length of a kept list for at most U units.
int64_t capacity(const Sel& s, int64_t U) {
  const int64_t k = keep_count_ppm(ratio_ppm(s.r), U);
  if (s.kind != SD_SEL_INIT_LOCAL_TOPK) return k;
  const int64_t c = static_cast<int64_t>(s.init) + s.local + k;
  return c < U ? c : U;
}

// Split plan of the attention pass for lists of up to k_max units: S splits
// per (sequence, KV head), each of E units, so that B * H_kv * S is about the
// block target; E is at least one 16-row chunk.
struct Split {
  int E;
  int S;
};

int64_t max_splits(const sdkv::Dims& d) {
  const int64_t bg = static_cast<int64_t>(d.B) * d.Hkv;
  int64_t s = ceil_div(target_blocks(), bg);
  return s < 1 ? 1 : (s > sdkv::kMaxSplits ? sdkv::kMaxSplits : s);
}

Split plan_split(const sdkv::Dims& d, int unit, int64_t k_max) {
  const int64_t kk = k_max < 1 ? 1 : k_max;
  int64_t E = ceil_div(kk, max_splits(d));
  if (unit == SD_UNIT_TOKEN) E = ceil_div(E, 16) * 16;
  return Split{static_cast<int>(E), static_cast<int>(ceil_div(kk, E))};
}

// Workspace regions (byte offsets).  The split count and the attention
// partials come first so that every entry point agrees on where they live.
struct Layout {
  size_t split_count, part_o, part_lse, attend_end, scores, logits, sel_idx, sel_count, msel,
      score_mm, topk_tmp, topk_cnt, total;
};

// Scratch of the many-block top-k (units beyond one block's registers).
bool multi_select(const sdkv::Dims& d, int unit) {
  return units_max(d, unit) > sdkv::kOneBlockTopkMax;
}

size_t select_ws_bytes(const sdkv::Dims& d, int unit) {
  return multi_select(d, unit) ? sdkv::msel_workspace_bytes(d.B, d.Hkv, units_max(d, unit)) : 0;
}

// The budget runs in one block per (b, g) up to kBudgetOneMax tokens, past
// that over many blocks (with the many-block top-k's scratch inside its own):
// the one-block kernel's time grows with the tokens, the many-block one's is
// mostly its launches, and the two meet near 8K tokens.
constexpr int kBudgetOneMax = 8192;

bool budget_multi(const sdkv::Dims& d, int unit, const Sel& s) {
  return s.kind == SD_SEL_MASS_BUDGET && units_max(d, unit) > kBudgetOneMax;
}

size_t select_ws_bytes(const sdkv::Dims& d, int unit, const Sel& s) {
  if (budget_multi(d, unit, s)) return sdkv::budget_multi_workspace_bytes(d, units_max(d, unit));
  return select_ws_bytes(d, unit);
}

// Partial min / max keys written by the token scorer for the many-block top-k.
int score_mm_parts(const sdkv::Dims& d) {
  const int per = sdkv::score_units_per_block(d.dtype, d.D);
  return (d.max_seq + per - 1) / per;
}

// The union of a selection keeps its top-k list in topk_tmp / topk_cnt.
Layout layout(const sdkv::Dims& d, int unit, const Sel& sel) {
  Layout L{};
  const int64_t S = max_splits(d);
  const int64_t bh = static_cast<int64_t>(d.B) * d.Hq;
  const int64_t bg = static_cast<int64_t>(d.B) * d.Hkv;
  const int64_t U = units_max(d, unit);
  const int64_t k_top = keep_count_ppm(ratio_ppm(sel.r), U);
  const int64_t k_max = capacity(sel, U);
  const bool uni = sel.kind == SD_SEL_INIT_LOCAL_TOPK;
  size_t off = 0;
  L.split_count = off; off = align_up(off + sizeof(int32_t));
  L.part_o = off;      off = align_up(off + sizeof(float) * bh * S * d.D);
  L.part_lse = off;    off = align_up(off + sizeof(float) * bh * S);
  L.attend_end = off;
  L.scores = off;      off = align_up(off + sizeof(float) * bg * U);
  L.logits = off;
  if (unit == SD_UNIT_TOKEN) off = align_up(off + sizeof(float) * bh * d.max_seq);
  L.sel_idx = off;     off = align_up(off + sizeof(int32_t) * bg * k_max);
  L.sel_count = off;   off = align_up(off + sizeof(int32_t) * bg);
  L.msel = off;        off = align_up(off + select_ws_bytes(d, unit, sel));
  L.score_mm = off;
  if (unit == SD_UNIT_TOKEN && multi_select(d, unit))
    off = align_up(off + sizeof(uint32_t) * 2 * bg * score_mm_parts(d));
  L.topk_tmp = off;
  if (uni) off = align_up(off + sizeof(int32_t) * bg * k_top);
  L.topk_cnt = off;
  if (uni) off = align_up(off + sizeof(int32_t) * bg);
  L.total = off;
  return L;
}

Layout layout(const sdkv::Dims& d, int unit, double r_kv) { return layout(d, unit, topk_sel(r_kv)); }

// Workspace of sd_select_units: the many-block top-k scratch, then (union)
// the top-k list and counts.
struct SelectLayout {
  size_t msel, tmp, cnt, total;
};

SelectLayout select_layout(const sdkv::Dims& d, int unit, const Sel& sel) {
  SelectLayout L{};
  const int64_t bg = static_cast<int64_t>(d.B) * d.Hkv;
  const int64_t k_top = keep_count_ppm(ratio_ppm(sel.r), units_max(d, unit));
  const bool uni = sel.kind == SD_SEL_INIT_LOCAL_TOPK;
  size_t off = 0;
  L.msel = off;
  if (sel.kind != SD_SEL_WINDOW) off = align_up(off + select_ws_bytes(d, unit, sel));
  L.tmp = off;
  if (uni) off = align_up(off + sizeof(int32_t) * bg * k_top);
  L.cnt = off;
  if (uni) off = align_up(off + sizeof(int32_t) * bg);
  L.total = off;
  return L;
}

size_t attend_ws_bytes(const sdkv::Dims& d) { return layout(d, SD_UNIT_PAGE, 1.0).attend_end; }

sd_status check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return SD_OK;
  if (!ws) return fail(SD_E_NULL, "workspace is NULL (%zu bytes needed)", need);
  if (reinterpret_cast<uintptr_t>(ws) % kAlign != 0)
    return fail(SD_E_WORKSPACE, "workspace must be %zu-byte aligned", kAlign);
  if (ws_bytes < need)
    return fail(SD_E_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed",
                ws_bytes, need);
  return SD_OK;
}

sd_status device_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return SD_OK;
  return fail(SD_E_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

char* at(void* ws, size_t off) { return static_cast<char*>(ws) + off; }

// ---- validated launches (arguments already checked) ----

sd_status do_score(const sdkv::Dims& d, const void* q, const void* k_pages, const void* bounds,
                   const int32_t* bt, const int32_t* sl, int unit, float* scores, float* logits,
                   hipStream_t st, uint32_t* score_mm = nullptr, bool logits_tm = false) {
  sdkv::ScoreArgs a{d, unit, q, k_pages, bounds, bt, sl, scores, logits, score_mm};
  a.logits_tm = logits_tm ? 1 : 0;
  return device_status(sdkv::launch_score(a, st), "score kernel launch");
}

sd_status do_score_compressed(const sdkv::Dims& d, const void* q, const float* ckeys,
                              const int32_t* sl, float* scores, hipStream_t st) {
  sdkv::CompressArgs a{};
  a.d = d;
  a.q = q;
  a.ckeys = const_cast<float*>(ckeys);
  a.seq_lens = sl;
  a.max_windows = sdkv::compressed_windows(d);
  a.unit_scores = scores;
  return device_status(sdkv::launch_score_compressed(a, st), "compressed scoring kernel launch");
}

// msel_ws: select_ws_bytes(d, unit) bytes (unused up to kMaxSelectOne units);
// score_mm: the token scorer's partial min / max keys, or NULL.
sd_status do_select(const sdkv::Dims& d, int unit, const int32_t* sl, const float* scores,
                    double r_kv, int32_t* sel_idx, int32_t* sel_count, void* msel_ws,
                    hipStream_t st, const uint32_t* score_mm = nullptr) {
  const int U = units_max(d, unit);
  const int R = ratio_ppm(r_kv);
  sdkv::SelectArgs a{d, unit, sl, scores, U, static_cast<int>(keep_count_ppm(R, U)), R,
                     sel_idx, sel_count};
  if (multi_select(d, unit))
    return device_status(
        sdkv::launch_select_multi(a, score_mm, score_mm ? score_mm_parts(d) : 0,
                                  score_mm ? sdkv::score_units_per_block(d.dtype, d.D) : 0,
                                  msel_ws, st),
        "select kernels launch");
  return device_status(sdkv::launch_select(a, st), "select kernel launch");
}

// Window list, or the union of the forced ranges with a top-k list.
sd_status do_structure(const sdkv::Dims& d, int unit, const int32_t* sl, const Sel& sel,
                       const int32_t* top, const int32_t* top_cnt, int top_stride,
                       int32_t* sel_idx, int32_t* sel_count, int cap, hipStream_t st) {
  sdkv::StructArgs a{};
  a.d = d;
  a.unit = unit;
  a.seq_lens = sl;
  a.kind = sel.kind == SD_SEL_WINDOW ? sdkv::kWindow : sdkv::kInitLocalTopk;
  a.R_ppm = ratio_ppm(sel.r);
  a.init_units = sel.init;
  a.local_units = sel.local;
  a.topk_idx = top;
  a.topk_count = top_cnt;
  a.topk_stride = top_stride;
  a.sel_idx = sel_idx;
  a.sel_count = sel_count;
  a.cap = cap;
  return device_status(sdkv::launch_structure(a, st), "structure kernel launch");
}

// How the attention kernel obtains a list without sel_idx: a window of the
// last keep_count units, or the forced ranges of an in-kernel union.
struct ListMode {
  bool window = false;
  int window_R = -1;
  int force_init = 0, force_local = 0;
};

// What the attention pass does with the logits: softmax (default),
// alpha-entmax against the thresholds tau (with stored logits), or write the
// logits of the attended tokens to logits_out and nothing else.
struct Weights {
  const float* tau = nullptr;
  float alpha_m1 = 0.f, beta = 0.f;
  float* logits_out = nullptr;
  bool logits_slots = false;  // AttendArgs::logits_slots
};

// Split-K attention partials.  Exactly one list source: sel_idx (list),
// unit_scores (top-k inside the kernel) or neither (identity, or a window).
sd_status do_partials(const sdkv::Dims& d, const void* q, const void* kp, const void* vp,
                      const int32_t* bt, const int32_t* sl, int unit, const int32_t* sel_idx,
                      const int32_t* sel_count, int k_max, const float* logits, void* ws,
                      hipStream_t st, const float* unit_scores = nullptr, int R_ppm = -1,
                      int32_t* sel_out = nullptr, int32_t* sel_count_out = nullptr,
                      int* S_out = nullptr, ListMode lm = ListMode{}, Weights wt = Weights{},
                      bool logits_tm = false) {
  const bool listed = sel_idx != nullptr || unit_scores != nullptr || lm.window;
  const int64_t kk = listed ? k_max : units_max(d, unit);
  const Split sp = plan_split(d, unit, kk);
  const Layout L = layout(d, unit, 1.0);
  sdkv::AttendArgs a{};
  a.d = d;
  a.unit = unit;
  a.q = q;
  a.k_pages = kp;
  a.v_pages = vp;
  a.block_table = bt;
  a.seq_lens = sl;
  a.sel_idx = sel_idx;
  a.sel_count = sel_count;
  a.k_max = listed ? k_max : 0;
  a.token_logits = logits;
  a.logits_tm = logits_tm ? 1 : 0;
  a.E = sp.E;
  a.S = sp.S;
  a.part_o = reinterpret_cast<float*>(at(ws, L.part_o));
  a.part_lse = reinterpret_cast<float*>(at(ws, L.part_lse));
  a.split_count = reinterpret_cast<int32_t*>(at(ws, L.split_count));
  a.unit_scores = unit_scores;
  a.R_ppm = R_ppm;
  a.sel_out = sel_out;
  a.sel_count_out = sel_count_out;
  a.force_init = lm.force_init;
  a.force_local = lm.force_local;
  if (lm.window) {
    a.window = 1;
    a.R_ppm = lm.window_R;
  }
  a.tau = wt.tau;
  a.alpha_m1 = wt.alpha_m1;
  a.beta = wt.beta;
  a.logits_out = wt.logits_out;
  a.logits_slots = wt.logits_slots ? 1 : 0;
  if (S_out) *S_out = sp.S;
  return device_status(sdkv::launch_attend(a, st), "attention kernel launch");
}

// S_known > 0: the split count of the attention launch just enqueued (saves
// the merge kernel a dependent read of the workspace header).
sd_status do_merge(const sdkv::Dims& d, float* out, float* lse, void* ws, hipStream_t st,
                   int S_known = 0) {
  const Layout L = layout(d, SD_UNIT_PAGE, 1.0);
  sdkv::MergeArgs a{};
  a.d = d;
  a.S_known = S_known;
  a.part_o = reinterpret_cast<const float*>(at(ws, L.part_o));
  a.part_lse = reinterpret_cast<const float*>(at(ws, L.part_lse));
  a.split_count = reinterpret_cast<const int32_t*>(at(ws, L.split_count));
  a.S_max = static_cast<int>(max_splits(d));
  a.out = out;
  a.lse = lse;
  return device_status(sdkv::launch_merge(a, st), "merge kernel launch");
}

// The plain top-k in token unit past one block's selection (bf16): the
// many-block top-k's placement runs inside the attention kernel, whose split
// j of (b, g) is then a range of kSliceUnits >> l units (l returned, the
// largest up to 3 that keeps NB << l within the splits the partials hold).
// -1: not this path (more slices than splits, or another selection).
int sliced_sub_log2(const sdkv::Dims& d, int unit, const Sel& sel) {
  if (unit != SD_UNIT_TOKEN || d.dtype != SD_BF16 || sel.kind != SD_SEL_TOPK || sel.r >= 1.0 ||
      !multi_select(d, unit))
    return -1;
  const int64_t NB = ceil_div(units_max(d, unit), sdkv::kSliceUnits);
  const int64_t S = max_splits(d);
  if (NB > S) return -1;
  int l = 0;
  while (l < 3 && (NB << (l + 1)) <= S) ++l;
  return l;
}

// Top-k selection and attention of that path: the histogram and candidate
// launches of the many-block top-k, then the attention with the placement
// (it writes the kept list to idx / cnt).
sd_status do_sliced_attend(const sdkv::Dims& d, const void* q, const void* kp, const void* vp,
                           const int32_t* bt, const int32_t* sl, double r_kv, int sub_log2,
                           const float* scores, const float* logits, const uint32_t* score_mm,
                           int32_t* idx, int32_t* cnt, void* msel_ws, void* ws, hipStream_t st,
                           int* S_out) {
  const int U = units_max(d, SD_UNIT_TOKEN);
  const int R = ratio_ppm(r_kv);
  const int k = static_cast<int>(keep_count_ppm(R, U));
  sdkv::SelectArgs sa{d, SD_UNIT_TOKEN, sl, scores, U, k, R, idx, cnt};
  sdkv::SliceSel ss;
  sd_status s;
  if ((s = device_status(sdkv::launch_select_multi_bins(sa, score_mm, score_mm_parts(d),
                                                         sdkv::score_units_per_block(d.dtype, d.D),
                                                         msel_ws, st, &ss),
                         "select kernels launch")) != SD_OK)
    return s;
  const Layout L = layout(d, SD_UNIT_TOKEN, 1.0);
  sdkv::AttendArgs a{};
  a.d = d;
  a.unit = SD_UNIT_TOKEN;
  a.q = q;
  a.k_pages = kp;
  a.v_pages = vp;
  a.block_table = bt;
  a.seq_lens = sl;
  a.k_max = k;
  a.R_ppm = R;
  a.token_logits = logits;
  a.logits_tm = 1;
  a.sl = ss;
  a.sub_log2 = sub_log2;
  a.S = ss.NB << sub_log2;
  // the expected kept units of a range (the resolve window only)
  const int64_t range = sdkv::kSliceUnits >> sub_log2;
  a.E = static_cast<int>(ceil_div(ceil_div(static_cast<int64_t>(k) * range, U), 16) * 16);
  a.part_o = reinterpret_cast<float*>(at(ws, L.part_o));
  a.part_lse = reinterpret_cast<float*>(at(ws, L.part_lse));
  a.split_count = reinterpret_cast<int32_t*>(at(ws, L.split_count));
  a.sel_out = idx;
  a.sel_count_out = cnt;
  *S_out = a.S;
  return device_status(sdkv::launch_attend(a, st), "attention kernel launch");
}

// Whether the top-k can run inside the attention kernel: page unit, bf16, at
// most kMaxSelectU pages per sequence, and a split slice that fits the
// kernel's LDS list.
bool fused_select(const sdkv::Dims& d, int unit, int k_max) {
  if (unit != SD_UNIT_PAGE || d.dtype != SD_BF16 || d.max_pages > sdkv::kMaxSelectU) return false;
  return plan_split(d, unit, k_max).E <= sdkv::kMaxSelectE;
}

// The kept lists of a selection (not a window) from unit scores: the top-k,
// or the top-k (kept in the workspace) merged with the forced ranges.  Rows
// of idx hold capacity(sel, U_max) entries; msel_ws holds
// select_ws_bytes(d, unit, sel) bytes.
sd_status do_select_list(const sdkv::Dims& d, int unit, const int32_t* sl, const float* scores,
                         const float* logits, const Sel& sel, int32_t* idx, int32_t* cnt,
                         void* msel_ws, int32_t* top_tmp, int32_t* top_cnt, hipStream_t s,
                         const uint32_t* score_mm = nullptr) {
  if (sel.kind == SD_SEL_TOPK)
    return do_select(d, unit, sl, scores, sel.r, idx, cnt, msel_ws, s, score_mm);
  if (sel.kind == SD_SEL_MASS_BUDGET) {
    sdkv::BudgetArgs a{};
    a.d = d;
    a.seq_lens = sl;
    a.scores = scores;
    a.logits = logits;
    a.U_max = units_max(d, unit);
    a.R_ppm = ratio_ppm(sel.r);
    a.k_max = static_cast<int>(keep_count_ppm(a.R_ppm, a.U_max));
    a.max_dropped = static_cast<float>(sel.dmax);
    a.sel_idx = idx;
    a.sel_count = cnt;
    if (budget_multi(d, unit, sel))
      return device_status(sdkv::launch_select_budget_multi(a, msel_ws, s),
                           "budget selection kernels launch");
    return device_status(sdkv::launch_select_budget(a, s), "budget selection kernel launch");
  }
  const int U = units_max(d, unit);
  const int k_top = static_cast<int>(keep_count_ppm(ratio_ppm(sel.r), U));
  sd_status st;
  if ((st = do_select(d, unit, sl, scores, sel.r, top_tmp, top_cnt, msel_ws, s, score_mm)) !=
      SD_OK)
    return st;
  return do_structure(d, unit, sl, sel, top_tmp, top_cnt, k_top, idx, cnt,
                      static_cast<int>(capacity(sel, U)), s);
}

// Page-unit selection + attention: fused when possible, else the kept lists
// then a listed attention.
sd_status do_select_attend(const sdkv::Dims& d, const void* q, const void* kp, const void* vp,
                           const int32_t* bt, const int32_t* sl, const float* scores,
                           const Sel& sel, float* out, float* lse, int32_t* sel_idx,
                           int32_t* sel_count, void* ws, hipStream_t s) {
  const int unit = SD_UNIT_PAGE;
  const Layout L = layout(d, unit, sel);
  const int k_max = static_cast<int>(capacity(sel, units_max(d, unit)));
  sd_status st;
  int S = 0;
  if (fused_select(d, unit, k_max)) {
    ListMode lm;
    lm.force_init = sel.init;
    lm.force_local = sel.local;
    if ((st = do_partials(d, q, kp, vp, bt, sl, unit, nullptr, nullptr, k_max, nullptr, ws, s,
                          scores, ratio_ppm(sel.r), sel_idx, sel_count, &S, lm)) != SD_OK)
      return st;
    return do_merge(d, out, lse, ws, s, S);
  }
  int32_t* idx = sel_idx ? sel_idx : reinterpret_cast<int32_t*>(at(ws, L.sel_idx));
  int32_t* cnt = sel_count ? sel_count : reinterpret_cast<int32_t*>(at(ws, L.sel_count));
  if ((st = do_select_list(d, unit, sl, scores, nullptr, sel, idx, cnt, at(ws, L.msel),
                           reinterpret_cast<int32_t*>(at(ws, L.topk_tmp)),
                           reinterpret_cast<int32_t*>(at(ws, L.topk_cnt)), s)) != SD_OK)
    return st;
  if ((st = do_partials(d, q, kp, vp, bt, sl, unit, idx, cnt, k_max, nullptr, ws, s, nullptr, -1,
                        nullptr, nullptr, &S)) != SD_OK)
    return st;
  return do_merge(d, out, lse, ws, s, S);
}

// The decode step under a selection (arguments and workspace size checked).
sd_status decode_impl(const sdkv::Dims& d, const void* q, const void* k_pages,
                      const void* v_pages, const void* page_bounds, const int32_t* block_table,
                      const int32_t* seq_lens, int unit, const Sel& sel, float* out, float* lse,
                      int32_t* sel_idx, int32_t* sel_count, void* ws, hipStream_t s) {
  const Layout L = layout(d, unit, sel);
  const int U = units_max(d, unit);
  const int k_max = static_cast<int>(capacity(sel, U));
  sd_status st;
  int S = 0;
  if (sel.r >= 1.0 && sel.kind != SD_SEL_MASS_BUDGET) {  // every unit: dense
    if ((st = do_partials(d, q, k_pages, v_pages, block_table, seq_lens, unit, nullptr, nullptr,
                          0, nullptr, ws, s, nullptr, -1, nullptr, nullptr, &S)) != SD_OK)
      return st;
    return do_merge(d, out, lse, ws, s, S);
  }
  if (sel.kind == SD_SEL_WINDOW) {  // no scores: the attention reads the window
    ListMode lm;
    lm.window = true;
    lm.window_R = ratio_ppm(sel.r);
    if (sel_idx &&
        (st = do_structure(d, unit, seq_lens, sel, nullptr, nullptr, 0, sel_idx, sel_count, k_max,
                           s)) != SD_OK)
      return st;
    if ((st = do_partials(d, q, k_pages, v_pages, block_table, seq_lens, unit, nullptr, nullptr,
                          k_max, nullptr, ws, s, nullptr, -1, nullptr, nullptr, &S, lm)) != SD_OK)
      return st;
    return do_merge(d, out, lse, ws, s, S);
  }
  float* scores = reinterpret_cast<float*>(at(ws, L.scores));
  float* logits = unit == SD_UNIT_TOKEN ? reinterpret_cast<float*>(at(ws, L.logits)) : nullptr;
  uint32_t* smm = unit == SD_UNIT_TOKEN && multi_select(d, unit)
                      ? reinterpret_cast<uint32_t*>(at(ws, L.score_mm))
                      : nullptr;
  // the logits stay inside this step unless the budget reads them: then
  // they are laid out token-major (whole-line writes, one piece per kept
  // token when the attention pass reads them)
  const bool tm = unit == SD_UNIT_TOKEN && sel.kind != SD_SEL_MASS_BUDGET;
  if (unit == SD_UNIT_PAGE && sel.scorer == SD_SCORER_COMPRESSED)
    st = do_score_compressed(d, q, static_cast<const float*>(page_bounds), seq_lens, scores, s);
  else
    st = do_score(d, q, k_pages, page_bounds, block_table, seq_lens, unit, scores, logits, s, smm,
                  tm);
  if (st != SD_OK) return st;
  if (unit == SD_UNIT_PAGE)
    return do_select_attend(d, q, k_pages, v_pages, block_table, seq_lens, scores, sel, out, lse,
                            sel_idx, sel_count, ws, s);
  int32_t* idx = sel_idx ? sel_idx : reinterpret_cast<int32_t*>(at(ws, L.sel_idx));
  int32_t* cnt = sel_count ? sel_count : reinterpret_cast<int32_t*>(at(ws, L.sel_count));
  const int sub = tm ? sliced_sub_log2(d, unit, sel) : -1;
  if (sub >= 0) {
    if ((st = do_sliced_attend(d, q, k_pages, v_pages, block_table, seq_lens, sel.r, sub, scores,
                               logits, smm, idx, cnt, at(ws, L.msel), ws, s, &S)) != SD_OK)
      return st;
    return do_merge(d, out, lse, ws, s, S);
  }
  if ((st = do_select_list(d, unit, seq_lens, scores, logits, sel, idx, cnt, at(ws, L.msel),
                           reinterpret_cast<int32_t*>(at(ws, L.topk_tmp)),
                           reinterpret_cast<int32_t*>(at(ws, L.topk_cnt)), s, smm)) != SD_OK)
    return st;
  if ((st = do_partials(d, q, k_pages, v_pages, block_table, seq_lens, unit, idx, cnt, k_max,
                        logits, ws, s, nullptr, -1, nullptr, nullptr, &S, ListMode{}, Weights{},
                        tm)) != SD_OK)
    return st;
  return do_merge(d, out, lse, ws, s, S);
}

// ---- alpha-entmax decode step ----

// Workspace of the entmax step: the decode-step layout, then (page unit) the
// logits of the attended tokens -- token unit keeps them where the token
// scorer writes them -- the thresholds, and the lse the merge writes (not
// reported: the entmax weights already sum to one).
struct EntLayout {
  Layout L;
  size_t logits, tau, lse, cand, cmax, ccnt, total;
  int nch;  // threshold chunks per head (0: one block per head)
};

// Most kept token slots of one head: the kept list's units (token unit) or
// their pages' rows (page unit); every unit when nothing is dropped.
int64_t entmax_slots(const sdkv::Dims& d, int unit, const Sel& sel) {
  const bool dense = sel.r >= 1.0 && sel.kind != SD_SEL_MASS_BUDGET;
  const int64_t units = dense ? units_max(d, unit) : capacity(sel, units_max(d, unit));
  return unit == SD_UNIT_PAGE ? units * d.P : units;
}

EntLayout ent_layout(const sdkv::Dims& d, int unit, const Sel& sel) {
  EntLayout E{};
  E.L = layout(d, unit, sel);
  const int64_t bh = static_cast<int64_t>(d.B) * d.Hq;
  size_t off = E.L.total;
  E.logits = E.L.logits;
  if (unit == SD_UNIT_PAGE) {
    E.logits = off;
    off = align_up(off + sizeof(float) * bh * d.max_seq);
  }
  E.tau = off;  off = align_up(off + sizeof(float) * bh);
  E.lse = off;  off = align_up(off + sizeof(float) * bh);
  const int64_t slots = entmax_slots(d, unit, sel);
  E.nch = slots > sdkv::kTauChunk ? static_cast<int>(ceil_div(slots, sdkv::kTauChunk)) : 0;
  const int64_t hc = bh * E.nch;
  E.cand = off; off = align_up(off + sizeof(float) * hc * sdkv::kTauChunkCap);
  E.cmax = off; off = align_up(off + sizeof(float) * hc);
  E.ccnt = off; off = align_up(off + sizeof(int32_t) * hc);
  E.total = off;
  return E;
}

// Selection as in decode_impl, then: the logits of the attended tokens (the
// token scorer's, or a logits-only pass of the attention kernel over the
// kept list), the threshold of every head over them, and the attention
// pass with entmax weights over the stored logits, merged by the LSE merge
// (each split reports the log of its weight sum; the merge divides the
// summed weighted values by the summed weights).
sd_status entmax_impl(const sdkv::Dims& d, const void* q, const void* k_pages,
                      const void* v_pages, const void* page_stats, const int32_t* block_table,
                      const int32_t* seq_lens, int unit, const Sel& sel, double alpha, float* out,
                      float* tau_out, int32_t* sel_idx, int32_t* sel_count, void* ws,
                      hipStream_t s) {
  const EntLayout E = ent_layout(d, unit, sel);
  const Layout& L = E.L;
  const int U = units_max(d, unit);
  const int k_max = static_cast<int>(capacity(sel, U));
  const bool dense = sel.r >= 1.0 && sel.kind != SD_SEL_MASS_BUDGET;
  float* logits = reinterpret_cast<float*>(at(ws, E.logits));
  float* tau = tau_out ? tau_out : reinterpret_cast<float*>(at(ws, E.tau));
  int32_t* idx = nullptr;
  int32_t* cnt = nullptr;
  sd_status st;
  bool have_logits = false;
  const float am1 = static_cast<float>(alpha - 1.0);
  const float beta = static_cast<float>(1.0 / (alpha - 1.0));
  // Page unit, top-k or union, where the attention kernel can select: the
  // logits-only pass selects the pages itself and writes the kept lists.
  const bool fused = !dense && unit == SD_UNIT_PAGE &&
                     (sel.kind == SD_SEL_TOPK || sel.kind == SD_SEL_INIT_LOCAL_TOPK) &&
                     fused_select(d, unit, k_max);
  // Logits written by the logits-only attention pass (every case but the
  // token scorer's) are laid out by kept slot on the matrix-core path: the
  // threshold kernel then reads them without the list and the block table,
  // and the entmax pass reads a split's logits as one run.
  const bool scorer_logits = unit == SD_UNIT_TOKEN && !dense && sel.kind != SD_SEL_WINDOW;
  const bool slots = d.dtype == SD_BF16 && !scorer_logits;
  if (!dense) {
    idx = sel_idx ? sel_idx : reinterpret_cast<int32_t*>(at(ws, L.sel_idx));
    cnt = sel_count ? sel_count : reinterpret_cast<int32_t*>(at(ws, L.sel_count));
    if (fused) {
      float* scores = reinterpret_cast<float*>(at(ws, L.scores));
      if (sel.scorer == SD_SCORER_COMPRESSED)
        st = do_score_compressed(d, q, static_cast<const float*>(page_stats), seq_lens, scores,
                                 s);
      else
        st = do_score(d, q, k_pages, page_stats, block_table, seq_lens, unit, scores, nullptr, s);
      if (st != SD_OK) return st;
      ListMode lm;
      lm.force_init = sel.init;
      lm.force_local = sel.local;
      Weights w;
      w.logits_out = logits;
      w.logits_slots = slots;
      if ((st = do_partials(d, q, k_pages, v_pages, block_table, seq_lens, unit, nullptr, nullptr,
                            k_max, nullptr, ws, s, scores, ratio_ppm(sel.r), idx, cnt, nullptr,
                            lm, w)) != SD_OK)
        return st;
      have_logits = true;
      st = SD_OK;
    } else if (sel.kind == SD_SEL_WINDOW) {
      st = do_structure(d, unit, seq_lens, sel, nullptr, nullptr, 0, idx, cnt, k_max, s);
    } else {
      float* scores = reinterpret_cast<float*>(at(ws, L.scores));
      uint32_t* smm = unit == SD_UNIT_TOKEN && multi_select(d, unit)
                          ? reinterpret_cast<uint32_t*>(at(ws, L.score_mm))
                          : nullptr;
      if (unit == SD_UNIT_PAGE && sel.scorer == SD_SCORER_COMPRESSED)
        st = do_score_compressed(d, q, static_cast<const float*>(page_stats), seq_lens, scores,
                                 s);
      else
        st = do_score(d, q, k_pages, page_stats, block_table, seq_lens, unit, scores,
                      unit == SD_UNIT_TOKEN ? logits : nullptr, s, smm);
      if (st != SD_OK) return st;
      have_logits = unit == SD_UNIT_TOKEN;
      st = do_select_list(d, unit, seq_lens, scores, have_logits ? logits : nullptr, sel, idx,
                          cnt, at(ws, L.msel), reinterpret_cast<int32_t*>(at(ws, L.topk_tmp)),
                          reinterpret_cast<int32_t*>(at(ws, L.topk_cnt)), s, smm);
    }
    if (st != SD_OK) return st;
  }
  if (!have_logits) {
    Weights w;
    w.logits_out = logits;
    w.logits_slots = slots;
    if ((st = do_partials(d, q, k_pages, v_pages, block_table, seq_lens, unit, idx, cnt, k_max,
                          nullptr, ws, s, nullptr, -1, nullptr, nullptr, nullptr, ListMode{},
                          w)) != SD_OK)
      return st;
  }
  sdkv::TauArgs ta{d, unit, seq_lens, block_table, idx, cnt, idx ? k_max : 0, logits, am1, beta,
                   tau, E.nch, reinterpret_cast<float*>(at(ws, E.cand)),
                   reinterpret_cast<float*>(at(ws, E.cmax)),
                   reinterpret_cast<int32_t*>(at(ws, E.ccnt))};
  ta.logits_slots = slots ? 1 : 0;
  if ((st = device_status(sdkv::launch_entmax_tau(ta, s), "entmax threshold kernel launch")) !=
      SD_OK)
    return st;
  Weights w;
  w.tau = tau;
  w.alpha_m1 = am1;
  w.beta = beta;
  w.logits_slots = slots;
  int S = 0;
  if ((st = do_partials(d, q, k_pages, v_pages, block_table, seq_lens, unit, idx, cnt, k_max,
                        logits, ws, s, nullptr, -1, nullptr, nullptr, &S, ListMode{}, w)) !=
      SD_OK)
    return st;
  return do_merge(d, out, reinterpret_cast<float*>(at(ws, E.lse)), ws, s, S);
}

sd_status check_alpha(double alpha) {
  if (!(std::isfinite(alpha) && alpha > 1.0 && alpha <= 2.0))
    return fail(SD_E_RATIO, "alpha must lie in (1, 2]");
  return SD_OK;
}

// The thresholds take at most kTauMaxChunks chunks of kTauChunk kept slots
// per head.
sd_status check_entmax_size(const EntLayout& E) {
  if (E.nch > sdkv::kTauMaxChunks)
    return fail(SD_E_UNSUPPORTED, "alpha-entmax takes at most %lld kept slots per head",
                static_cast<long long>(sdkv::kTauMaxChunks) * sdkv::kTauChunk);
  return SD_OK;
}

// Shared checks of the attention entry points.
sd_status check_attend_args(const sdkv::Dims& d, int32_t unit, const void* q, const void* k_pages,
                            const void* v_pages, const int32_t* block_table,
                            const int32_t* seq_lens, const int32_t* sel_idx,
                            const int32_t* sel_count, int32_t k_max,
                            const float* token_logits) {
  sd_status st;
  if ((st = check_unit(unit)) != SD_OK) return st;
  if (!q || !v_pages || !block_table || !seq_lens)
    return fail(SD_E_NULL, "q, v_pages, block_table and seq_lens are required");
  if (!token_logits && !k_pages) return fail(SD_E_NULL, "k_pages is required");
  if (token_logits && unit != SD_UNIT_TOKEN)
    return fail(SD_E_SHAPE, "token_logits is only read in token unit");
  if (sel_idx) {
    if (!sel_count) return fail(SD_E_NULL, "sel_count is required with sel_idx");
    if (k_max < 1 || k_max > units_max(d, unit))
      return fail(SD_E_SHAPE, "k_max %d outside [1, %d]", k_max, units_max(d, unit));
  }
  return SD_OK;
}

}  // namespace

extern "C" {

int32_t sd_keep_count(double r_kv, int32_t num_units) {
  if (!std::isfinite(r_kv) || r_kv <= 0.0 || num_units < 1) return -1;
  return static_cast<int32_t>(keep_count_ppm(ratio_ppm(r_kv), num_units));
}

sd_status sd_workspace_bytes(const sd_shape* shape, int32_t unit, double r_kv,
                             size_t* bytes_host) {
  sdkv::Dims d;
  sd_status st;
  if ((st = check_shape(shape, &d)) != SD_OK) return st;
  if ((st = check_unit(unit)) != SD_OK) return st;
  if ((st = check_ratio(r_kv)) != SD_OK) return st;
  if (!bytes_host) return fail(SD_E_NULL, "bytes_host is NULL");
  *bytes_host = layout(d, unit, r_kv).total;
  return ok();
}

sd_status sd_update_page_bounds(const sd_shape* shape, const void* k_pages,
                                const int32_t* block_table, const int32_t* seq_lens,
                                const int32_t* pages, int32_t n_pages, void* page_bounds,
                                void* stream) {
  sdkv::Dims d;
  sd_status st;
  if ((st = check_shape(shape, &d)) != SD_OK) return st;
  if (!k_pages || !block_table || !seq_lens || !page_bounds)
    return fail(SD_E_NULL, "k_pages, block_table, seq_lens and page_bounds are required");
  if (pages && n_pages < 0) return fail(SD_E_SHAPE, "n_pages (%d) must be >= 0", n_pages);
  if (pages && n_pages == 0) return ok();  // an empty list: nothing to enqueue
  sdkv::BoundsArgs a{d, k_pages, block_table, seq_lens, page_bounds};
  a.pages = pages;
  a.n_pages = pages ? n_pages : 0;
  if ((st = device_status(sdkv::launch_page_bounds(a, static_cast<hipStream_t>(stream)),
                          "page bounds kernel launch")) != SD_OK)
    return st;
  return ok();
}

sd_status sd_append_page_bounds(const sd_shape* shape, const void* k_pages,
                                const int32_t* block_table, const int32_t* seq_lens,
                                const int32_t* appended, int32_t max_appended,
                                void* page_bounds, void* stream) {
  sdkv::Dims d;
  sd_status st;
  if ((st = check_shape(shape, &d)) != SD_OK) return st;
  if (!k_pages || !block_table || !seq_lens || !appended || !page_bounds)
    return fail(SD_E_NULL,
                "k_pages, block_table, seq_lens, appended and page_bounds are required");
  if (max_appended < 1 || max_appended > d.max_seq)
    return fail(SD_E_SHAPE, "max_appended (%d) outside [1, max_seq_len = %d]", max_appended,
                d.max_seq);
  sdkv::BoundsArgs a{d, k_pages, block_table, seq_lens, page_bounds};
  a.appended = appended;
  a.max_appended = max_appended;
  if ((st = device_status(sdkv::launch_page_bounds(a, static_cast<hipStream_t>(stream)),
                          "page bounds append kernel launch")) != SD_OK)
    return st;
  return ok();
}

sd_status sd_score_pages(const sd_shape* shape, const void* q, const void* k_pages,
                         const void* page_bounds, const int32_t* block_table,
                         const int32_t* seq_lens, int32_t unit, float* unit_scores,
                         float* token_logits, void* stream) {
  sdkv::Dims d;
  sd_status st;
  if ((st = check_shape(shape, &d)) != SD_OK) return st;
  if ((st = check_unit(unit)) != SD_OK) return st;
  if (!q || !block_table || !seq_lens || !unit_scores)
    return fail(SD_E_NULL, "q, block_table, seq_lens and unit_scores are required");
  if (unit == SD_UNIT_PAGE && !page_bounds)
    return fail(SD_E_NULL, "page unit scoring reads page_bounds");
  if (unit == SD_UNIT_TOKEN && (!k_pages || !token_logits))
    return fail(SD_E_NULL, "token unit scoring reads k_pages and writes token_logits");
  if ((st = do_score(d, q, k_pages, page_bounds, block_table, seq_lens, unit, unit_scores,
                     token_logits, static_cast<hipStream_t>(stream))) != SD_OK)
    return st;
  return ok();
}

sd_status sd_select_topk(const sd_shape* shape, int32_t unit, const int32_t* seq_lens,
                         const float* unit_scores, double r_kv, int32_t* sel_idx,
                         int32_t* sel_count, void* ws, size_t ws_bytes, void* stream) {
  sdkv::Dims d;
  sd_status st;
  if ((st = check_shape(shape, &d)) != SD_OK) return st;
  if ((st = check_unit(unit)) != SD_OK) return st;
  if ((st = check_ratio(r_kv)) != SD_OK) return st;
  if (!seq_lens || !unit_scores || !sel_idx || !sel_count)
    return fail(SD_E_NULL, "seq_lens, unit_scores, sel_idx and sel_count are required");
  if ((st = check_ws(ws, ws_bytes, select_ws_bytes(d, unit))) != SD_OK) return st;
  if ((st = do_select(d, unit, seq_lens, unit_scores, r_kv, sel_idx, sel_count, ws,
                      static_cast<hipStream_t>(stream))) != SD_OK)
    return st;
  return ok();
}

sd_status sd_attend_partials(const sd_shape* shape, const void* q, const void* k_pages,
                             const void* v_pages, const int32_t* block_table,
                             const int32_t* seq_lens, int32_t unit, const int32_t* sel_idx,
                             const int32_t* sel_count, int32_t k_max, const float* token_logits,
                             const float* unit_scores, double r_kv, int32_t* sel_out,
                             int32_t* sel_count_out, void* ws, size_t ws_bytes, void* stream) {
  sdkv::Dims d;
  sd_status st;
  if ((st = check_shape(shape, &d)) != SD_OK) return st;
  if ((st = check_attend_args(d, unit, q, k_pages, v_pages, block_table, seq_lens, sel_idx,
                              sel_count, k_max, token_logits)) != SD_OK)
    return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (unit_scores) {
    if (sel_idx) return fail(SD_E_SHAPE, "give either sel_idx or unit_scores, not both");
    if (unit != SD_UNIT_PAGE) return fail(SD_E_SHAPE, "in-kernel top-k is page unit only");
    if ((st = check_ratio(r_kv)) != SD_OK) return st;
    if ((sel_out == nullptr) != (sel_count_out == nullptr))
      return fail(SD_E_NULL, "sel_out and sel_count_out are given together or not at all");
    const int km = static_cast<int>(keep_count_ppm(ratio_ppm(r_kv), units_max(d, unit)));
    if (!fused_select(d, unit, km))
      return fail(SD_E_UNSUPPORTED,
                  "in-kernel top-k needs bf16 data, <= %d pages per sequence and <= %d kept "
                  "pages per split",
                  sdkv::kMaxSelectU, sdkv::kMaxSelectE);
    if ((st = check_ws(ws, ws_bytes, attend_ws_bytes(d))) != SD_OK) return st;
    if ((st = do_partials(d, q, k_pages, v_pages, block_table, seq_lens, unit, nullptr, nullptr,
                          km, nullptr, ws, s, unit_scores, ratio_ppm(r_kv), sel_out,
                          sel_count_out)) != SD_OK)
      return st;
    return ok();
  }
  if (sel_out || sel_count_out) return fail(SD_E_SHAPE, "sel_out is written by in-kernel top-k only");
  if ((st = check_ws(ws, ws_bytes, attend_ws_bytes(d))) != SD_OK) return st;
  if ((st = do_partials(d, q, k_pages, v_pages, block_table, seq_lens, unit, sel_idx, sel_count,
                        k_max, token_logits, ws, s)) != SD_OK)
    return st;
  return ok();
}

sd_status sd_merge_splits(const sd_shape* shape, float* out, float* lse, void* ws,
                          size_t ws_bytes, void* stream) {
  sdkv::Dims d;
  sd_status st;
  if ((st = check_shape(shape, &d)) != SD_OK) return st;
  if (!out || !lse) return fail(SD_E_NULL, "out and lse are required");
  if ((st = check_ws(ws, ws_bytes, attend_ws_bytes(d))) != SD_OK) return st;
  if ((st = do_merge(d, out, lse, ws, static_cast<hipStream_t>(stream))) != SD_OK) return st;
  return ok();
}

sd_status sd_attend_splitk(const sd_shape* shape, const void* q, const void* k_pages,
                           const void* v_pages, const int32_t* block_table,
                           const int32_t* seq_lens, int32_t unit, const int32_t* sel_idx,
                           const int32_t* sel_count, int32_t k_max, const float* token_logits,
                           float* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  sdkv::Dims d;
  sd_status st;
  if ((st = check_shape(shape, &d)) != SD_OK) return st;
  if ((st = check_attend_args(d, unit, q, k_pages, v_pages, block_table, seq_lens, sel_idx,
                              sel_count, k_max, token_logits)) != SD_OK)
    return st;
  if (!out || !lse) return fail(SD_E_NULL, "out and lse are required");
  if ((st = check_ws(ws, ws_bytes, attend_ws_bytes(d))) != SD_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int S = 0;
  if ((st = do_partials(d, q, k_pages, v_pages, block_table, seq_lens, unit, sel_idx, sel_count,
                        k_max, token_logits, ws, s, nullptr, -1, nullptr, nullptr, &S)) != SD_OK)
    return st;
  if ((st = do_merge(d, out, lse, ws, s, S)) != SD_OK) return st;
  return ok();
}

sd_status sd_select_attend(const sd_shape* shape, const void* q, const void* k_pages,
                           const void* v_pages, const int32_t* block_table,
                           const int32_t* seq_lens, const float* unit_scores, double r_kv,
                           float* out, float* lse, int32_t* sel_idx, int32_t* sel_count,
                           void* ws, size_t ws_bytes, void* stream) {
  sdkv::Dims d;
  sd_status st;
  if ((st = check_shape(shape, &d)) != SD_OK) return st;
  if ((st = check_ratio(r_kv)) != SD_OK) return st;
  if (!q || !k_pages || !v_pages || !block_table || !seq_lens || !unit_scores || !out || !lse)
    return fail(SD_E_NULL,
                "q, k_pages, v_pages, block_table, seq_lens, unit_scores, out and lse are required");
  if ((sel_idx == nullptr) != (sel_count == nullptr))
    return fail(SD_E_NULL, "sel_idx and sel_count are given together or not at all");
  if ((st = check_ws(ws, ws_bytes, layout(d, SD_UNIT_PAGE, r_kv).total)) != SD_OK) return st;
  if ((st = do_select_attend(d, q, k_pages, v_pages, block_table, seq_lens, unit_scores,
                             topk_sel(r_kv), out, lse, sel_idx, sel_count, ws,
                             static_cast<hipStream_t>(stream))) != SD_OK)
    return st;
  return ok();
}

sd_status sd_decode_step(const sd_shape* shape, const void* q, const void* k_pages,
                         const void* v_pages, const void* page_bounds,
                         const int32_t* block_table, const int32_t* seq_lens, int32_t unit,
                         double r_kv, float* out, float* lse, int32_t* sel_idx,
                         int32_t* sel_count, void* ws, size_t ws_bytes, void* stream) {
  sdkv::Dims d;
  sd_status st;
  if ((st = check_shape(shape, &d)) != SD_OK) return st;
  if ((st = check_unit(unit)) != SD_OK) return st;
  if ((st = check_ratio(r_kv)) != SD_OK) return st;
  if (!q || !k_pages || !v_pages || !block_table || !seq_lens || !out || !lse)
    return fail(SD_E_NULL,
                "q, k_pages, v_pages, block_table, seq_lens, out and lse are required");
  const bool dense = r_kv >= 1.0;
  if (!dense && unit == SD_UNIT_PAGE && !page_bounds)
    return fail(SD_E_NULL, "page unit selection reads page_bounds");
  if ((sel_idx == nullptr) != (sel_count == nullptr))
    return fail(SD_E_NULL, "sel_idx and sel_count are given together or not at all");
  if ((st = check_ws(ws, ws_bytes, layout(d, unit, r_kv).total)) != SD_OK) return st;
  if ((st = decode_impl(d, q, k_pages, v_pages, page_bounds, block_table, seq_lens, unit,
                        topk_sel(r_kv), out, lse, sel_idx, sel_count, ws,
                        static_cast<hipStream_t>(stream))) != SD_OK)
    return st;
  return ok();
}

sd_status sd_update_compressed_keys(const sd_shape* shape, const void* k_pages,
                                    const int32_t* block_table, const int32_t* seq_lens,
                                    float* compressed_keys, void* stream) {
  sdkv::Dims d;
  sd_status st;
  if ((st = check_shape(shape, &d)) != SD_OK) return st;
  if (!k_pages || !block_table || !seq_lens || !compressed_keys)
    return fail(SD_E_NULL, "k_pages, block_table, seq_lens and compressed_keys are required");
  sdkv::CompressArgs a{};
  a.d = d;
  a.k_pages = k_pages;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.ckeys = compressed_keys;
  a.max_windows = sdkv::compressed_windows(d);
  if ((st = device_status(sdkv::launch_compress_keys(a, static_cast<hipStream_t>(stream)),
                          "compressed keys kernel launch")) != SD_OK)
    return st;
  return ok();
}

sd_status sd_score_compressed(const sd_shape* shape, const void* q, const float* compressed_keys,
                              const int32_t* seq_lens, float* unit_scores, void* stream) {
  sdkv::Dims d;
  sd_status st;
  if ((st = check_shape(shape, &d)) != SD_OK) return st;
  if (!q || !compressed_keys || !seq_lens || !unit_scores)
    return fail(SD_E_NULL, "q, compressed_keys, seq_lens and unit_scores are required");
  if ((st = do_score_compressed(d, q, compressed_keys, seq_lens, unit_scores,
                                static_cast<hipStream_t>(stream))) != SD_OK)
    return st;
  return ok();
}

int32_t sd_selection_capacity(const sd_selection* sel, int32_t num_units) {
  Sel v;
  if (num_units < 1 || check_selection(sel, &v) != SD_OK) return -1;
  return static_cast<int32_t>(capacity(v, num_units));
}

sd_status sd_workspace_bytes_sel(const sd_shape* shape, int32_t unit, const sd_selection* sel,
                                 size_t* bytes_host) {
  sdkv::Dims d;
  Sel v;
  sd_status st;
  if ((st = check_shape(shape, &d)) != SD_OK) return st;
  if ((st = check_unit(unit)) != SD_OK) return st;
  if ((st = check_selection(sel, &v)) != SD_OK) return st;
  if (!bytes_host) return fail(SD_E_NULL, "bytes_host is NULL");
  const size_t a = layout(d, unit, v).total, b = select_layout(d, unit, v).total;
  *bytes_host = a > b ? a : b;
  return ok();
}

sd_status sd_select_units(const sd_shape* shape, int32_t unit, const int32_t* seq_lens,
                          const float* unit_scores, const float* token_logits,
                          const sd_selection* sel, int32_t* sel_idx, int32_t* sel_count, void* ws,
                          size_t ws_bytes, void* stream) {
  sdkv::Dims d;
  Sel v;
  sd_status st;
  if ((st = check_shape(shape, &d)) != SD_OK) return st;
  if ((st = check_unit(unit)) != SD_OK) return st;
  if ((st = check_selection(sel, &v)) != SD_OK) return st;
  if (!seq_lens || !sel_idx || !sel_count || (!unit_scores && v.kind != SD_SEL_WINDOW))
    return fail(SD_E_NULL, "seq_lens, sel_idx, sel_count and (unless a window) unit_scores "
                           "are required");
  if ((st = check_budget(d, unit, v)) != SD_OK) return st;
  if (v.kind == SD_SEL_MASS_BUDGET && !token_logits)
    return fail(SD_E_NULL, "the dropped-mass budget reads token_logits");
  const SelectLayout SL = select_layout(d, unit, v);
  if ((st = check_ws(ws, ws_bytes, SL.total)) != SD_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int cap = static_cast<int>(capacity(v, units_max(d, unit)));
  if (v.kind == SD_SEL_WINDOW)
    st = do_structure(d, unit, seq_lens, v, nullptr, nullptr, 0, sel_idx, sel_count, cap, s);
  else
    st = do_select_list(d, unit, seq_lens, unit_scores, token_logits, v, sel_idx, sel_count,
                        at(ws, SL.msel), reinterpret_cast<int32_t*>(at(ws, SL.tmp)),
                        reinterpret_cast<int32_t*>(at(ws, SL.cnt)), s);
  if (st != SD_OK) return st;
  return ok();
}

sd_status sd_decode_step_sel(const sd_shape* shape, const void* q, const void* k_pages,
                             const void* v_pages, const void* page_bounds,
                             const int32_t* block_table, const int32_t* seq_lens, int32_t unit,
                             const sd_selection* sel, float* out, float* lse, int32_t* sel_idx,
                             int32_t* sel_count, void* ws, size_t ws_bytes, void* stream) {
  sdkv::Dims d;
  Sel v;
  sd_status st;
  if ((st = check_shape(shape, &d)) != SD_OK) return st;
  if ((st = check_unit(unit)) != SD_OK) return st;
  if ((st = check_selection(sel, &v)) != SD_OK) return st;
  if (!q || !k_pages || !v_pages || !block_table || !seq_lens || !out || !lse)
    return fail(SD_E_NULL,
                "q, k_pages, v_pages, block_table, seq_lens, out and lse are required");
  if ((st = check_budget(d, unit, v)) != SD_OK) return st;
  if (v.r < 1.0 && v.kind != SD_SEL_WINDOW && unit == SD_UNIT_PAGE && !page_bounds)
    return fail(SD_E_NULL, "page unit selection reads page_bounds");
  if ((sel_idx == nullptr) != (sel_count == nullptr))
    return fail(SD_E_NULL, "sel_idx and sel_count are given together or not at all");
  if ((st = check_ws(ws, ws_bytes, layout(d, unit, v).total)) != SD_OK) return st;
  if ((st = decode_impl(d, q, k_pages, v_pages, page_bounds, block_table, seq_lens, unit, v, out,
                        lse, sel_idx, sel_count, ws, static_cast<hipStream_t>(stream))) != SD_OK)
    return st;
  return ok();
}

sd_status sd_workspace_bytes_entmax(const sd_shape* shape, int32_t unit,
                                    const sd_selection* sel, size_t* bytes_host) {
  sdkv::Dims d;
  Sel v;
  sd_status st;
  if ((st = check_shape(shape, &d)) != SD_OK) return st;
  if ((st = check_unit(unit)) != SD_OK) return st;
  if ((st = check_selection(sel, &v)) != SD_OK) return st;
  if (!bytes_host) return fail(SD_E_NULL, "bytes_host is NULL");
  const EntLayout E = ent_layout(d, unit, v);
  if ((st = check_entmax_size(E)) != SD_OK) return st;
  *bytes_host = E.total;
  return ok();
}

sd_status sd_decode_step_entmax(const sd_shape* shape, const void* q, const void* k_pages,
                                const void* v_pages, const void* page_stats,
                                const int32_t* block_table, const int32_t* seq_lens,
                                int32_t unit, const sd_selection* sel, double alpha, float* out,
                                float* tau, int32_t* sel_idx, int32_t* sel_count, void* ws,
                                size_t ws_bytes, void* stream) {
  sdkv::Dims d;
  Sel v;
  sd_status st;
  if ((st = check_shape(shape, &d)) != SD_OK) return st;
  if ((st = check_unit(unit)) != SD_OK) return st;
  if ((st = check_selection(sel, &v)) != SD_OK) return st;
  if ((st = check_alpha(alpha)) != SD_OK) return st;
  if (!q || !k_pages || !v_pages || !block_table || !seq_lens || !out)
    return fail(SD_E_NULL, "q, k_pages, v_pages, block_table, seq_lens and out are required");
  if ((st = check_budget(d, unit, v)) != SD_OK) return st;
  if (v.r < 1.0 && v.kind != SD_SEL_WINDOW && unit == SD_UNIT_PAGE && !page_stats)
    return fail(SD_E_NULL, "page unit selection reads page_stats");
  if ((sel_idx == nullptr) != (sel_count == nullptr))
    return fail(SD_E_NULL, "sel_idx and sel_count are given together or not at all");
  const EntLayout E = ent_layout(d, unit, v);
  if ((st = check_entmax_size(E)) != SD_OK) return st;
  if ((st = check_ws(ws, ws_bytes, E.total)) != SD_OK) return st;
  if ((st = entmax_impl(d, q, k_pages, v_pages, page_stats, block_table, seq_lens, unit, v, alpha,
                        out, tau, sel_idx, sel_count, ws, static_cast<hipStream_t>(stream))) !=
      SD_OK)
    return st;
  return ok();
}

sd_status sd_dropped_mass(const sd_shape* shape, const int32_t* seq_lens,
                          const int32_t* block_table, const float* token_logits,
                          const int32_t* sel_idx, const int32_t* sel_count, int32_t k_max,
                          float* delta, void* stream) {
  sdkv::Dims d;
  sd_status st;
  if ((st = check_shape(shape, &d)) != SD_OK) return st;
  if (!seq_lens || !block_table || !token_logits || !sel_idx || !sel_count || !delta)
    return fail(SD_E_NULL, "seq_lens, block_table, token_logits, sel_idx, sel_count and delta "
                           "are required");
  if (k_max < 1 || k_max > d.max_seq)
    return fail(SD_E_SHAPE, "k_max %d outside [1, %d]", k_max, d.max_seq);
  if (d.max_seq > sdkv::kMaxDropSeq)
    return fail(SD_E_UNSUPPORTED, "the dropped mass takes at most %d tokens per sequence",
                sdkv::kMaxDropSeq);
  sdkv::DropArgs a{d, seq_lens, block_table, token_logits, sel_idx, sel_count, k_max, delta};
  if ((st = device_status(sdkv::launch_dropped_mass(a, static_cast<hipStream_t>(stream)),
                          "dropped mass kernel launch")) != SD_OK)
    return st;
  return ok();
}

const char* sd_last_error(void) { return g_err; }

// For sd_decode_step_noalloc (noalloc.hip): a status with its message, as
// sd_last_error() reports it.  Not exported.
sd_status sdkv_fail_noalloc(sd_status st, const char* msg) { return fail(st, "%s", msg); }

}  // extern "C"
