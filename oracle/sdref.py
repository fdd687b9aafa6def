"""fp64 reference for one decode step of sparse GQA attention.

TEST INFRASTRUCTURE (see the package docstring): only tests/, smoke() and the
bench's cpu_baseline leg may call this module.

What is computed, step by step, for one sequence b and one KV head g (the G
query heads h with h // G == g share that KV head and one selection):

1. logits      s[h, t] = scale * <q[h], K[g, t]> for every valid key t < n
2. dense       p = softmax(s[h]);  o = sum_t p_t V[g, t];  lse = log sum_t e^s
3. unit scores token unit: sigma[t] = max_h s[h, t]
               page unit:  sigma[u] = max_h scale * sum_c max(q[h,c] kmin[u,c],
                                                          q[h,c] kmax[u,c])
               with kmin/kmax taken over the valid tokens of page u
4. keep count  k = clamp(ceil(R * U / 10^6), 1, U), R = r_KV in integer parts
               per million; r_KV >= 1 keeps every unit
5. top-k       the k largest sigma, equal scores going to the lower unit id,
               reported in ascending unit order, plus the score gap at k
6. sparse      softmax attention of each head over the valid tokens of the
               kept units only (renormalised over that set)
7. dropped     delta[h] = dense softmax mass of the tokens not kept

Sources (page title, then the part of the page):
* [Cross/cards] "Where Activation Sparsity and KV-Cache Sparsity Cross in LLM
  Decoding", cards view. Pre-hoc sparsity abstract: the dropped mass delta of
  the discarded entries. EntmaxKV abstract: pages are scored against the
  query from light per-page statistics before they are loaded, candidates
  are selected, attention runs on the selection, and the output error is
  governed by delta.
* [Cross/list] the same title, list view. Abstract: attention-scored KV
  selection; dense and sparse decoding read the cache through one split-K
  kernel. Tables 4 and 16: a keep ratio of 1 turns a branch off.
* [Mass] "Attention-Mass Condensation for Sparse Decoding", second abstract:
  dense attention, a top-k token support, attention recomputed on the support.
* [SparDA] "SparDA: Sparse Decoupled Attention ..." summary, Section 3.1:
  full attention is computed over the attended blocks only; GQA query heads
  share one KV head and one block selection. Appendix C: 64-token blocks.

Readings where the pages leave a step open:
the page bound form and max-over-group aggregation (step 3), consecutive
head groups g = h // G, ceil in integer ppm for k (step 4), ties to the lower
index and ascending output (step 5), scale 1/sqrt(d) on scores too.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np


# ----------------------------------------------------------------------------
# stored values -> fp64
# ----------------------------------------------------------------------------

def widen(stored: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 copy of stored values.

    ``dtype == "f32"``: the array holds IEEE binary32 values.
    ``dtype == "bf16"``: the array holds bfloat16 bit patterns as uint16; a
    bfloat16 is the upper half of a binary32, so shifting the bits up by 16
    gives the same number as a binary32, which fp64 holds exactly.
    """
    if dtype == "f32":
        return np.asarray(stored, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(stored, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# ----------------------------------------------------------------------------
# step 1-2: logits and softmax attention
# ----------------------------------------------------------------------------

def group_logits(q_group: np.ndarray, K: np.ndarray, scale: float) -> np.ndarray:
    """Step 1 for the G query heads of one KV head.

    q_group: [G, d] queries of the heads h = g*G .. g*G+G-1.
    K:       [n, d] the valid keys of KV head g.
    Returns s: [G, n], s[i, t] = scale * sum_c q_group[i, c] * K[t, c].
    """
    return scale * (np.asarray(q_group, np.float64) @ np.asarray(K, np.float64).T)


def logits(q: np.ndarray, K: np.ndarray, scale: float) -> np.ndarray:
    """Step 1 for all heads of one sequence: q [H_q, d], K [H_kv, n, d] -> s [H_q, n].

    Query head h reads KV head h // G with G = H_q / H_kv (consecutive groups).
    """
    H_q, H_kv = q.shape[0], K.shape[0]
    if H_q % H_kv:
        raise ValueError("H_q must be a multiple of H_kv")
    G = H_q // H_kv
    s = np.empty((H_q, K.shape[1]), dtype=np.float64)
    for h in range(H_q):
        s[h] = scale * (np.asarray(K[h // G], np.float64) @ np.asarray(q[h], np.float64))
    return s


def attention(s: np.ndarray, V: np.ndarray, tokens: np.ndarray | None = None):
    """Step 2 (and step 6 when ``tokens`` is given) for one query head.

    s: [n] logits, V: [n, d] values, tokens: ascending positions to attend to
    (None = all n).  Returns (o [d], lse) with o = sum_t p_t V_t,
    p = softmax(s restricted to tokens), lse = log sum_t exp(s_t).
    """
    s = np.asarray(s, np.float64)
    V = np.asarray(V, np.float64)
    if tokens is not None:
        s = s[tokens]
        V = V[tokens]
    if s.size == 0:
        raise ValueError("attention over an empty set")
    m = s.max()
    w = np.exp(s - m)
    Z = w.sum()
    return (w @ V) / Z, m + math.log(Z)


def split_partial(s: np.ndarray, V: np.ndarray, tokens: np.ndarray):
    """One split of split-K attention ([Cross/list] Abstract: dense and sparse
    decoding through one split-K kernel): the attention of one query head
    over the split's own ``tokens`` alone, as (o_j [d], lse_j).  An empty
    split is (0, -inf), which weighs nothing in the merge."""
    tokens = np.asarray(tokens, dtype=np.int64)
    if tokens.size == 0:
        return np.zeros(np.asarray(V).shape[1]), -math.inf
    return attention(s, V, tokens)


def merge_splits(parts):
    """Log-sum-exp merge of split partials [(o_j, lse_j), ...] in fp64:
    M = max_j lse_j, w_j = exp(lse_j - M), o = sum_j w_j o_j / sum_j w_j,
    lse = M + log sum_j w_j.  Splits with lse_j = -inf contribute nothing;
    if every split is empty the result is (0, -inf), an empty sequence."""
    lses = np.array([p[1] for p in parts], dtype=np.float64)
    os_ = np.array([p[0] for p in parts], dtype=np.float64)
    if lses.size == 0 or not np.any(np.isfinite(lses)):
        return np.zeros(os_.shape[1] if os_.ndim == 2 else 0), -math.inf
    M = lses.max()
    w = np.exp(lses - M)
    Z = w.sum()
    return (w @ os_) / Z, M + math.log(Z)


def split_attention(s: np.ndarray, V: np.ndarray, splits):
    """Split-K attention of one head: ``splits`` is a list of token-index
    arrays (any partition of the attended tokens, empty parts allowed); each
    is attended alone (``split_partial``) and the partials are merged
    (``merge_splits``).  The partition is free: the result equals one-shot
    attention over the union up to rounding."""
    return merge_splits([split_partial(s, V, t) for t in splits])


def dropped_mass(s: np.ndarray, tokens: np.ndarray) -> float:
    """Step 7: delta = sum of the dense softmax weights of the positions NOT in
    ``tokens`` ([Cross/cards], pre-hoc sparsity abstract), summed directly over
    the dropped positions rather than as 1 minus the kept mass."""
    s = np.asarray(s, np.float64)
    m = s.max()
    w = np.exp(s - m)
    dropped = np.ones(s.shape[0], dtype=bool)
    dropped[np.asarray(tokens, dtype=np.int64)] = False
    return float(w[dropped].sum() / w.sum())


# ----------------------------------------------------------------------------
# step 3: unit scores
# ----------------------------------------------------------------------------

def num_units(n: int, unit: str, page_size: int) -> int:
    """U: n tokens in token unit; ceil(n / P) pages in page unit."""
    if unit == "token":
        return n
    if unit == "page":
        return -(-n // page_size)
    raise ValueError(f"unknown unit {unit!r}")


def page_bounds(K: np.ndarray, page_size: int):
    """Per-page key statistics of one KV head ([Cross/cards], EntmaxKV abstract:
    light page statistics, known before a page is loaded).

    K: [n, d] valid keys.  Page u holds tokens u*P .. min((u+1)*P, n) - 1; the
    bounds are the channel-wise min and max over those valid tokens only.
    Returns kmin, kmax: [U, d].
    """
    K = np.asarray(K, np.float64)
    n, d = K.shape
    U = num_units(n, "page", page_size)
    kmin = np.empty((U, d))
    kmax = np.empty((U, d))
    for u in range(U):
        rows = K[u * page_size: min((u + 1) * page_size, n)]
        kmin[u] = rows.min(axis=0)
        kmax[u] = rows.max(axis=0)
    return kmin, kmax


def page_scores(q_group: np.ndarray, kmin: np.ndarray, kmax: np.ndarray,
                scale: float) -> np.ndarray:
    """Step 3, page unit, for one KV head.

    sigma[u] = max over the G heads of scale * sum_c max(q_c*kmin[u,c], q_c*kmax[u,c]).
    For every head and every valid token t of page u, <q, K_t> <= sum_c
    max(q_c kmin_c, q_c kmax_c), so sigma[u] bounds the page's largest logit.
    """
    q_group = np.asarray(q_group, np.float64)
    G = q_group.shape[0]
    per_head = np.empty((G, kmin.shape[0]))
    for i in range(G):
        qi = q_group[i]
        per_head[i] = scale * np.maximum(qi * kmin, qi * kmax).sum(axis=1)
    return per_head.max(axis=0)


# Compressed-key block scoring ([SparDA] Section 3.1: a parameter-free
# selector mean-pools the keys into overlapping compressed representations,
# sums the per-head relevance over the GQA group and max-pools it to the
# block score; Appendix C: kernel 32, stride 16, 64-token blocks).
COMPRESS_KERNEL = 32
COMPRESS_STRIDE = 16


def compressed_keys(K: np.ndarray) -> np.ndarray:
    """Window j of one KV head: the mean of the valid keys 16 j .. 16 j + 31
    (fewer at the end of the sequence), for j < ceil(n / 16).  Returns [J, d]."""
    K = np.asarray(K, np.float64)
    n = K.shape[0]
    J = -(-n // COMPRESS_STRIDE)
    out = np.empty((J, K.shape[1]))
    for j in range(J):
        out[j] = K[j * COMPRESS_STRIDE: min(j * COMPRESS_STRIDE + COMPRESS_KERNEL, n)].mean(axis=0)
    return out


def compressed_page_scores(q_group: np.ndarray, ckeys: np.ndarray, page_size: int,
                           scale: float) -> np.ndarray:
    """Page score from the compressed keys, for one KV head: the relevance of
    window j is the sum over the group's heads of scale * <q_h, c_j>, and page
    u (tokens u P .. u P + P - 1) scores the max over the windows that start
    inside it, j = u P / 16 .. (u + 1) P / 16 - 1 (j < J).  A 64-token page
    pools four windows; a 16-token page takes the one window that starts on
    it (covering it and the next page)."""
    q_group = np.asarray(q_group, np.float64)
    rel = scale * (ckeys @ q_group.T).sum(axis=1)          # [J]
    J = rel.shape[0]
    per = page_size // COMPRESS_STRIDE
    U = -(-J // per)
    return np.array([rel[u * per: min((u + 1) * per, J)].max() for u in range(U)])


def token_scores(s_group: np.ndarray) -> np.ndarray:
    """Step 3, token unit, for one KV head: sigma[t] = max over the G heads of s[h, t]."""
    return np.asarray(s_group, np.float64).max(axis=0)


# ----------------------------------------------------------------------------
# step 4-5: keep count and top-k
# ----------------------------------------------------------------------------

def keep_count(r_kv: float, U: int) -> int:
    """Step 4: number of units kept under keep ratio r_KV.

    r_KV >= 1 keeps all U units ([Cross/list] Tables 4 and 16: ratio 1 turns
    the branch off).  Otherwise R = floor(r_KV * 10^6 + 1/2) parts per million
    and k = ceil(R * U / 10^6) in integer arithmetic, clamped to [1, U].
    """
    if not math.isfinite(r_kv) or r_kv <= 0.0:
        raise ValueError("r_KV must be finite and > 0")
    if U < 1:
        raise ValueError("need at least one unit")
    if r_kv >= 1.0:
        return U
    R = int(math.floor(r_kv * 1e6 + 0.5))
    k = -((-R * U) // 1_000_000)
    return min(max(k, 1), U)


def select_topk(sigma: np.ndarray, k: int):
    """Step 5: exact top-k by a stable sort.

    Units are ordered by decreasing score, equal scores by increasing unit id
    (so ties go to the lower index); the first k are kept and returned in
    ascending unit order.  gap = sigma of the k-th kept unit minus sigma of
    the best dropped unit (inf when nothing is dropped).
    """
    sigma = np.asarray(sigma, np.float64)
    if not np.all(np.isfinite(sigma)):
        raise ValueError("scores must be finite")
    U = sigma.shape[0]
    if not 1 <= k <= U:
        raise ValueError("k out of range")
    order = np.lexsort((np.arange(U), -sigma))
    kept = np.sort(order[:k])
    gap = float(sigma[order[k - 1]] - sigma[order[k]]) if k < U else math.inf
    return kept, gap


# ----------------------------------------------------------------------------
# structured index sets (instead of step 5)
# ----------------------------------------------------------------------------

@dataclass(frozen=True)
class Selection:
    """Which units a decode step keeps.

    kind "topk": step 5 with k = keep_count(r_kv, U).
    kind "window": the k = keep_count(r_kv, U) most recent units, the KV-window
        baseline of [Cross/list] Table 3 (a window of 30% of the context).
    kind "init_local_topk": the union of the first ``init_units`` units, the
        last ``local_units`` units and the step-5 top-k of all U units
        ([SparDA] Section 3.1: initial, local sliding-window and top-k blocks;
        Appendix A: the selected set is B_init U B_local U f_top(scores, k)).
    kind "mass_budget" (token unit): the shortest prefix of the step-5 order
        whose dropped dense mass is at most ``max_dropped`` for every head of
        the group, capped at keep_count(r_kv, U) units ([Cross/cards],
        pre-hoc sparsity abstract: the dropped mass delta is controlled in
        advance).
    """
    kind: str = "topk"
    r_kv: float = 0.3
    init_units: int = 0
    local_units: int = 0
    max_dropped: float = 0.0


def window_set(U: int, r_kv: float) -> np.ndarray:
    """The k = keep_count(r_kv, U) most recent units U-k .. U-1, ascending."""
    k = keep_count(r_kv, U)
    return np.arange(U - k, U, dtype=np.int64)


def init_local_topk_set(sigma: np.ndarray, r_kv: float, init_units: int,
                        local_units: int) -> np.ndarray:
    """B_init U B_local U top-k(sigma, keep_count(r_kv, U)), ascending.

    The top-k ranks all U units (scores of initial and local units included),
    so the three parts may overlap and the set holds between k and
    min(U, init + local + k) units.
    """
    sigma = np.asarray(sigma, np.float64)
    U = sigma.shape[0]
    if init_units < 0 or local_units < 0:
        raise ValueError("init_units and local_units must be >= 0")
    top, _ = select_topk(sigma, keep_count(r_kv, U))
    keep = np.zeros(U, dtype=bool)
    keep[:min(init_units, U)] = True
    keep[max(U - local_units, 0):] = True
    keep[top] = True
    return np.flatnonzero(keep).astype(np.int64)


def mass_budget_count(s_group: np.ndarray, sigma: np.ndarray, max_dropped: float,
                      k_cap: int) -> int:
    """Token unit: the smallest k such that keeping the first k units of the
    step-5 order (decreasing sigma, equal scores to the lower id) leaves a
    dense softmax mass of at most ``max_dropped`` outside the set for every
    head h of the group, capped at k_cap.

    s_group [G, n] logits, sigma [n] = max over the group.  The dropped mass
    after k units is the sum of p_h over the units after position k, summed
    directly (a suffix sum), as in step 7.
    """
    s = np.asarray(s_group, np.float64)
    sigma = np.asarray(sigma, np.float64)
    n = sigma.shape[0]
    if not 1 <= k_cap <= n:
        raise ValueError("k_cap out of range")
    if not (math.isfinite(max_dropped) and max_dropped >= 0.0):
        raise ValueError("max_dropped must be finite and >= 0")
    order = np.lexsort((np.arange(n), -sigma))
    m = s.max(axis=1, keepdims=True)
    w = np.exp(s - m)
    p = w / w.sum(axis=1, keepdims=True)
    # dropped[h, k] = sum_{j >= k} p[h, order[j]] for k = 0..n (dropped[:, n] = 0)
    tail = np.zeros((s.shape[0], n + 1))
    tail[:, :n] = np.cumsum(p[:, order][:, ::-1], axis=1)[:, ::-1]
    worst = tail.max(axis=0)                     # over the heads
    ok = np.flatnonzero(worst[1:] <= max_dropped)  # k = 1..n
    k = int(ok[0]) + 1 if ok.size else n
    return min(k, k_cap)


def selected_units(sigma: np.ndarray, sel: Selection, s_group=None) -> np.ndarray:
    """The kept units of one (sequence, KV head) under ``sel``, ascending
    (``s_group``, the group's logits, is needed by kind "mass_budget")."""
    U = np.asarray(sigma).shape[0]
    if sel.kind == "topk":
        return select_topk(sigma, keep_count(sel.r_kv, U))[0]
    if sel.kind == "window":
        return window_set(U, sel.r_kv)
    if sel.kind == "init_local_topk":
        return init_local_topk_set(sigma, sel.r_kv, sel.init_units, sel.local_units)
    if sel.kind == "mass_budget":
        if s_group is None:
            raise ValueError("mass_budget needs the group's logits")
        k = mass_budget_count(s_group, sigma, sel.max_dropped, keep_count(sel.r_kv, U))
        return select_topk(sigma, k)[0]
    raise ValueError(f"unknown selection kind {sel.kind!r}")


def selection_capacity(sel: Selection, U: int) -> int:
    """Most units ``sel`` keeps for a sequence of at most U units (the row
    length of a kept-list buffer)."""
    k = keep_count(sel.r_kv, U)
    if sel.kind in ("topk", "window", "mass_budget"):
        return k
    return min(U, sel.init_units + sel.local_units + k)


def unit_tokens(kept: np.ndarray, unit: str, page_size: int, n: int) -> np.ndarray:
    """Token positions covered by the kept units, ascending ([SparDA] Section
    3.1: attention over the attended blocks only).  A page contributes its
    valid tokens u*P .. min((u+1)*P, n) - 1."""
    kept = np.asarray(kept, dtype=np.int64)
    if unit == "token":
        return kept
    parts = [np.arange(u * page_size, min((u + 1) * page_size, n)) for u in kept]
    return np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)


# ----------------------------------------------------------------------------
# steps 1-7 for one selection instance and for a batch
# ----------------------------------------------------------------------------

@dataclass
class GroupResult:
    """Everything the oracle reports for one (sequence, KV head)."""
    sigma: np.ndarray       # [U] unit scores
    k: int                  # keep count
    kept: np.ndarray        # [k] kept unit ids, ascending
    gap: float              # score gap at the k-th unit
    out_dense: np.ndarray   # [G, d]
    lse_dense: np.ndarray   # [G]
    out_sparse: np.ndarray  # [G, d]
    lse_sparse: np.ndarray  # [G]
    delta: np.ndarray       # [G] dropped dense mass
    kmin: np.ndarray | None = None   # [U, d] page unit only
    kmax: np.ndarray | None = None


def group_step(q_group, K, V, *, unit: str, page_size: int, r_kv: float,
               scale: float, kept_override=None, selection: Selection | None = None,
               scorer: str = "bounds") -> GroupResult:
    """Steps 1-7 for one sequence and one KV head.

    q_group [G, d], K [n, d], V [n, d]: fp64 values of the valid tokens.
    ``kept_override`` (ascending unit ids) replaces step 5's set, so that an
    output can be recomputed on another selection of the same size.
    ``selection`` (kind other than "topk") replaces step 5's set by a
    structured one; k and gap still describe the step-5 top-k.  ``scorer``
    "compressed" scores pages from the compressed keys instead of the page
    bounds (page unit).
    """
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    n = K.shape[0]
    s = group_logits(q_group, K, scale)
    G = s.shape[0]
    kmin = kmax = None
    if unit == "page" and scorer == "compressed":
        sigma = compressed_page_scores(q_group, compressed_keys(K), page_size, scale)
    elif unit == "page":
        kmin, kmax = page_bounds(K, page_size)
        sigma = page_scores(q_group, kmin, kmax, scale)
    elif unit == "token":
        sigma = token_scores(s)
    else:
        raise ValueError(f"unknown unit {unit!r}")
    U = sigma.shape[0]
    k = keep_count(r_kv, U)
    kept, gap = select_topk(sigma, k)
    if selection is not None and selection.kind != "topk":
        if selection.kind == "mass_budget" and unit != "token":
            raise ValueError("mass_budget is token unit only")
        kept = selected_units(sigma, selection, s)
    if kept_override is not None:
        kept = np.asarray(kept_override, dtype=np.int64)
    tokens = unit_tokens(kept, unit, page_size, n)
    d = V.shape[1]
    out_d = np.empty((G, d)); lse_d = np.empty(G)
    out_s = np.empty((G, d)); lse_s = np.empty(G)
    delta = np.empty(G)
    for i in range(G):
        out_d[i], lse_d[i] = attention(s[i], V)
        out_s[i], lse_s[i] = attention(s[i], V, tokens)
        delta[i] = dropped_mass(s[i], tokens)
    return GroupResult(sigma, k, kept, gap, out_d, lse_d, out_s, lse_s, delta, kmin, kmax)


def decode_step(q, K, V, seq_lens, *, dtype: str, unit: str, page_size: int,
                r_kv: float, scale: float | None = None, groups=None,
                selection: Selection | None = None, scorer: str = "bounds"):
    """Steps 1-7 for a batch.

    q: [B, H_q, d]; K, V: [B, H_kv, n_max, d] stored values (float32, or
    uint16 bfloat16 bits when dtype == "bf16"); seq_lens: [B] valid lengths.
    ``groups``: optional iterable of (b, g) pairs to evaluate (default all).
    Returns {(b, g): GroupResult}.
    """
    B, H_q, d = q.shape
    H_kv = K.shape[1]
    G = H_q // H_kv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if groups is None:
        groups = [(b, g) for b in range(B) for g in range(H_kv)]
    res = {}
    for b, g in groups:
        n = int(seq_lens[b])
        qg = widen(q[b, g * G:(g + 1) * G], dtype)
        Kg = widen(K[b, g, :n], dtype)
        Vg = widen(V[b, g, :n], dtype)
        res[(b, g)] = group_step(qg, Kg, Vg, unit=unit, page_size=page_size,
                                 r_kv=r_kv, scale=scale, selection=selection, scorer=scorer)
    return res
