"""fp64 reference for alpha-entmax attention over a kept set.

TEST INFRASTRUCTURE (see the package docstring): only tests/, smoke() and the
bench's cpu_baseline leg may call this module.

Source: [Cross/cards] "Where Activation Sparsity and KV-Cache Sparsity Cross
in LLM Decoding", cards view, EntmaxKV abstract.  alpha-entmax gives exact
zeros, so sparse decoding becomes support recovery: if the selected
candidates hold the entmax support, sparse decoding is exact; otherwise the
output error is governed by the dropped probability mass delta.  The method
scores pages from light statistics, selects candidates and runs sparse
entmax attention on them.

The map (alpha-entmax of the logits z of one head, 1 < alpha <= 2):

    x_t = (alpha - 1) z_t
    p_t = max(x_t - tau, 0) ** (1 / (alpha - 1)),   tau such that sum_t p_t = 1

which is the Tsallis-regularised argmax; alpha = 2 is sparsemax and
alpha -> 1 tends to softmax.  tau is found by bisection on
f(tau) = sum_t max(x_t - tau, 0) ** (1 / (alpha - 1)) - 1, which decreases in
tau, with f(max x - 1) >= 0 (the largest term alone is 1) and
f(max x - n ** (1 - alpha)) <= 0 (each of the n terms is at most 1 / n).

Readings where the pages leave a step open (both sides implement these):
* alpha is a parameter; 1.5 is the default (the pages do not print it).
* The logits are the scaled ones of the softmax path, z = scale * q . K.
* Sparse entmax attention over a kept set T recomputes tau over T alone and
  attends with those weights (as the softmax path renormalises over T).
* The selection (scores, keep count, top-k, structured sets) is the softmax
  path's, unchanged; only the attention map differs.
* The bisection ends when the bracket no longer shrinks; the weights are then
  divided by their sum (the usual last step of a bisection entmax), which
  changes them by at most a few ulps in fp64.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

from . import sdref


def _check_alpha(alpha: float) -> None:
    if not (math.isfinite(alpha) and 1.0 < alpha <= 2.0):
        raise ValueError("alpha must lie in (1, 2]")


def entmax_threshold(z: np.ndarray, alpha: float, max_iter: int = 400) -> float:
    """tau of alpha-entmax(z) by bisection (module docstring)."""
    _check_alpha(alpha)
    z = np.asarray(z, np.float64)
    if z.size == 0:
        raise ValueError("entmax of an empty vector")
    if not np.all(np.isfinite(z)):
        raise ValueError("logits must be finite")
    beta = 1.0 / (alpha - 1.0)
    x = (alpha - 1.0) * z
    xm = float(x.max())
    lo = xm - 1.0
    hi = xm - float(z.size) ** (1.0 - alpha)

    def f(tau):
        return float(np.sum(np.maximum(x - tau, 0.0) ** beta)) - 1.0

    for _ in range(max_iter):
        mid = 0.5 * (lo + hi)
        if not lo < mid < hi:
            break
        if f(mid) >= 0.0:
            lo = mid
        else:
            hi = mid
    return lo


def entmax(z: np.ndarray, alpha: float) -> tuple[np.ndarray, float]:
    """alpha-entmax(z): (p, tau) with p = max((alpha-1) z - tau, 0) ** (1/(alpha-1)),
    divided by its sum."""
    z = np.asarray(z, np.float64)
    tau = entmax_threshold(z, alpha)
    p = np.maximum((alpha - 1.0) * z - tau, 0.0) ** (1.0 / (alpha - 1.0))
    return p / p.sum(), tau


def entmax_attention(s: np.ndarray, V: np.ndarray, alpha: float, tokens=None):
    """Entmax attention of one query head: (o [d], tau, support size).

    s: [n] logits, V: [n, d]; ``tokens`` (ascending positions, None = all):
    tau is recomputed over that set and the other positions weigh nothing.
    """
    s = np.asarray(s, np.float64)
    V = np.asarray(V, np.float64)
    if tokens is not None:
        tokens = np.asarray(tokens, dtype=np.int64)
        s = s[tokens]
        V = V[tokens]
    p, tau = entmax(s, alpha)
    return p @ V, tau, int(np.count_nonzero(p))


def entmax_dropped_mass(s: np.ndarray, tokens, alpha: float) -> float:
    """delta: the dense entmax mass of the positions NOT in ``tokens``, summed
    directly over them ([Cross/cards], EntmaxKV abstract).  It is 0 exactly
    when the kept set holds the support."""
    p, _ = entmax(s, alpha)
    dropped = np.ones(p.shape[0], dtype=bool)
    dropped[np.asarray(tokens, dtype=np.int64)] = False
    return float(p[dropped].sum())


@dataclass
class EntmaxGroupResult:
    """Entmax outputs for one (sequence, KV head); the selection is the
    softmax path's (sdref.group_step steps 1-5)."""
    sigma: np.ndarray       # [U] unit scores
    k: int                  # keep count
    kept: np.ndarray        # kept unit ids, ascending
    gap: float              # score gap at the k-th unit
    out_dense: np.ndarray   # [G, d] entmax over every valid token
    tau_dense: np.ndarray   # [G]
    out_sparse: np.ndarray  # [G, d] entmax over the kept tokens, tau recomputed
    tau_sparse: np.ndarray  # [G]
    delta: np.ndarray       # [G] dense entmax mass outside the kept tokens
    support: np.ndarray     # [G] dense support sizes


def group_step(q_group, K, V, *, unit: str, page_size: int, r_kv: float, scale: float,
               alpha: float = 1.5, kept_override=None,
               selection: sdref.Selection | None = None,
               scorer: str = "bounds") -> EntmaxGroupResult:
    """Scoring and selection as sdref.group_step, then entmax attention of
    every head of the group over all valid tokens and over the kept ones."""
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    n = K.shape[0]
    s = sdref.group_logits(q_group, K, scale)
    G = s.shape[0]
    if unit == "page" and scorer == "compressed":
        sigma = sdref.compressed_page_scores(q_group, sdref.compressed_keys(K), page_size, scale)
    elif unit == "page":
        kmin, kmax = sdref.page_bounds(K, page_size)
        sigma = sdref.page_scores(q_group, kmin, kmax, scale)
    elif unit == "token":
        sigma = sdref.token_scores(s)
    else:
        raise ValueError(f"unknown unit {unit!r}")
    U = sigma.shape[0]
    k = sdref.keep_count(r_kv, U)
    kept, gap = sdref.select_topk(sigma, k)
    if selection is not None and selection.kind != "topk":
        kept = sdref.selected_units(sigma, selection, s)
    if kept_override is not None:
        kept = np.asarray(kept_override, dtype=np.int64)
    tokens = sdref.unit_tokens(kept, unit, page_size, n)
    d = V.shape[1]
    out_d = np.empty((G, d)); tau_d = np.empty(G)
    out_s = np.empty((G, d)); tau_s = np.empty(G)
    delta = np.empty(G)
    support = np.empty(G, dtype=np.int64)
    for i in range(G):
        p, tau_d[i] = entmax(s[i], alpha)
        out_d[i] = p @ V
        support[i] = np.count_nonzero(p)
        out_s[i], tau_s[i], _ = entmax_attention(s[i], V, alpha, tokens)
        dropped = np.ones(n, dtype=bool)
        dropped[tokens] = False
        delta[i] = float(p[dropped].sum())
    return EntmaxGroupResult(sigma, k, kept, gap, out_d, tau_d, out_s, tau_s, delta, support)
