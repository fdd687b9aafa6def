"""Pins of the oracle's structured index sets (the KV window, initial +
local + top-k blocks, and the dropped-mass budget).

* window: it is the suffix of the context, so a window of every unit is dense
  attention exactly, and a page-unit window covers exactly the last tokens;
  on the planted-needle inputs it drops far more mass than the top-k of the
  same size (the pages' Table 3: a window misses most needles);
* union: an O(n^2) rank count plus the two forced ranges, over random and
  tied scores for n <= 40; no forced units is the plain top-k; forced ranges
  that cover every unit give dense attention; a superset of the top-k drops
  no more mass and obeys the 2 * delta * max|V| bound; the capacity bounds
  the set size, and matches the 64-token-block configuration of the pages
  (1 initial block, a 2048-token window, 96 top-k blocks);
* dropped-mass budget: with one head it is the textbook top-p count (exact
  sums); in general the shortest step-5 prefix whose step-7 dropped mass is
  within the target for every head (and one unit fewer is not); 0 and 1 as
  targets, monotonicity and the cap; whole decode steps report delta within
  the target.
"""

import math

import numpy as np
import pytest

import kvsynth
from oracle import sdref

Sel = sdref.Selection


def _rank_count_union(sigma, k, init, local):
    n = len(sigma)
    out = []
    for u in range(n):
        ahead = sum(1 for v in range(n) if sigma[v] > sigma[u] or (sigma[v] == sigma[u] and v < u))
        if u < init or u >= n - local or ahead < k:
            out.append(u)
    return np.array(out, dtype=np.int64)


@pytest.mark.parametrize("seed", range(24))
def test_union_matches_rank_count(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(1, 41))
    sigma = (rng.integers(-2, 3, size=n).astype(float) if seed % 2 else rng.standard_normal(n))
    for r in (0.01, 0.2, 0.5, 1.0):
        k = sdref.keep_count(r, n)
        for init, local in ((0, 0), (1, 0), (0, 3), (2, 5), (n, 0), (0, n + 4)):
            got = sdref.init_local_topk_set(sigma, r, init, local)
            np.testing.assert_array_equal(got, _rank_count_union(sigma, k, init, local))
            cap = sdref.selection_capacity(Sel("init_local_topk", r, init, local), n)
            assert k <= len(got) <= cap <= n


def test_union_without_forced_units_is_topk():
    rng = np.random.default_rng(7)
    sigma = rng.standard_normal(300)
    for r in (0.05, 0.3):
        top, _ = sdref.select_topk(sigma, sdref.keep_count(r, 300))
        np.testing.assert_array_equal(sdref.init_local_topk_set(sigma, r, 0, 0), top)
        np.testing.assert_array_equal(sdref.selected_units(sigma, Sel("topk", r)), top)


def test_window_is_the_suffix():
    for U, r in ((1, 0.3), (10, 0.3), (1000, 0.3), (2048, 0.05), (7, 1.0)):
        w = sdref.window_set(U, r)
        k = sdref.keep_count(r, U)
        assert len(w) == k and w[0] == U - k and w[-1] == U - 1
        assert np.all(np.diff(w) == 1)


def test_page_window_covers_last_tokens():
    n, P = 1000, 64            # 16 pages, the last one holds 40 tokens
    U = sdref.num_units(n, "page", P)
    kept = sdref.window_set(U, 0.25)            # 4 pages
    toks = sdref.unit_tokens(kept, "page", P, n)
    np.testing.assert_array_equal(toks, np.arange(12 * P, n))


@pytest.mark.parametrize("unit,P", [("token", 16), ("page", 16), ("page", 64)])
def test_full_window_and_full_union_are_dense(unit, P):
    rec = kvsynth.RECIPES["l8b"].with_(seq_len=700, unit=unit, page_size=P, num_q_heads=8,
                                       num_kv_heads=2)
    w = kvsynth.generate(rec)
    U = sdref.num_units(700, unit, P)
    for sel in (Sel("window", 1.0), Sel("init_local_topk", 0.01, 3, U)):
        res = sdref.decode_step(w.q, w.K, w.V, w.seq_lens, dtype="bf16", unit=unit,
                                page_size=P, r_kv=0.01, selection=sel)
        for gr in res.values():
            np.testing.assert_array_equal(gr.kept, np.arange(U))
            np.testing.assert_array_equal(gr.out_sparse, gr.out_dense)
            assert np.all(gr.delta == 0.0)


def test_union_drops_no_more_than_topk_and_obeys_bound():
    rec = kvsynth.RECIPES["l70b"].with_(seq_len=6000)
    w = kvsynth.generate(rec)
    r = 0.05
    top = sdref.decode_step(w.q, w.K, w.V, w.seq_lens, dtype="bf16", unit="page", page_size=64,
                            r_kv=r, groups=[(0, 0), (0, 5)])
    uni = sdref.decode_step(w.q, w.K, w.V, w.seq_lens, dtype="bf16", unit="page", page_size=64,
                            r_kv=r, groups=[(0, 0), (0, 5)],
                            selection=Sel("init_local_topk", r, 1, 8))
    for key in top:
        a, b = top[key], uni[key]
        assert set(a.kept.tolist()) <= set(b.kept.tolist())
        assert {0} | set(range(len(a.sigma) - 8, len(a.sigma))) <= set(b.kept.tolist())
        assert np.all(b.delta <= a.delta + 1e-15)
        V = sdref.widen(w.V[0, key[1], :6000], "bf16")
        vmax = np.linalg.norm(V, axis=1).max()
        for i in range(rec.group):
            assert np.linalg.norm(b.out_sparse[i] - b.out_dense[i]) <= 2 * b.delta[i] * vmax + 1e-12


def test_window_misses_needles():
    """Token unit on the tiny needle inputs: the window keeps about 25% of the
    planted keys (they are spread uniformly) and drops several times the mass
    that the top-k of the same size drops."""
    w = kvsynth.generate(kvsynth.RECIPES["tiny"])
    kw = dict(dtype="f32", unit="token", page_size=16, r_kv=0.25)
    top = sdref.decode_step(w.q, w.K, w.V, w.seq_lens, **kw)[(0, 0)]
    win = sdref.decode_step(w.q, w.K, w.V, w.seq_lens, selection=Sel("window", 0.25), **kw)[(0, 0)]
    planted = w.salient[(0, 0)]
    assert len(win.kept) == len(top.kept) == 256
    assert np.isin(planted, win.kept).mean() < 0.45
    assert np.isin(planted, top.kept).mean() > 0.9
    assert np.all(win.delta > 1.5 * top.delta)


def test_capacity_of_the_block_configuration():
    """64-token blocks at 1M context: 1 initial block, a 2048-token local
    window (32 blocks) and 96 top-k blocks keep at most 129 blocks."""
    U = (1 << 20) // 64
    r = 96 / U
    assert sdref.keep_count(r, U) == 96
    sel = Sel("init_local_topk", r, 1, 2048 // 64)
    assert sdref.selection_capacity(sel, U) == 129
    assert sdref.selection_capacity(Sel("window", 0.3), 2048) == 615
    assert sdref.selection_capacity(Sel("init_local_topk", 0.5, 10, 10), 12) == 12


def test_unknown_kind_rejected():
    with pytest.raises(ValueError):
        sdref.selected_units(np.zeros(4), Sel("sliding", 0.5))
    with pytest.raises(ValueError):
        sdref.init_local_topk_set(np.zeros(4), 0.5, -1, 0)


# ---------------------------------------------------------------- dropped-mass budget

def _nucleus_count(p, max_dropped):
    """Textbook top-p: sort the probabilities in decreasing order and keep the
    shortest prefix whose complement sums (exactly, math.fsum) to at most
    max_dropped."""
    q = np.sort(np.asarray(p))[::-1]
    for k in range(1, len(q) + 1):
        if math.fsum(q[k:]) <= max_dropped:
            return k
    return len(q)


@pytest.mark.parametrize("seed", range(10))
def test_budget_one_head_is_top_p(seed):
    """With one head, sigma is the head's own logit, so the budget is the
    nucleus (top-p, p = 1 - max_dropped) count of its softmax."""
    rng = np.random.default_rng(300 + seed)
    n = int(rng.integers(5, 400))
    s = rng.standard_normal((1, n)) * rng.uniform(0.5, 4.0)
    p = np.exp(s[0] - s[0].max())
    p /= p.sum()
    for dstar in rng.uniform(0.0, 0.6, size=6):
        k = sdref.mass_budget_count(s, s[0], float(dstar), n)
        # skip thresholds within rounding of a prefix sum
        q = np.sort(p)[::-1]
        if np.min(np.abs(np.cumsum(q[::-1])[::-1] - dstar)) < 1e-12:
            continue
        assert k == _nucleus_count(p, float(dstar))


@pytest.mark.parametrize("seed", range(12))
def test_budget_is_smallest_topk_within_delta(seed):
    """Every head: the kept top-k drops <= max_dropped, and one unit fewer
    would drop more for some head (step 5's set, step 7's mass)."""
    rng = np.random.default_rng(400 + seed)
    G = int(rng.integers(1, 5))
    n = int(rng.integers(2, 60))
    s = rng.standard_normal((G, n)) * 2.0
    if seed % 3 == 0:
        s = np.round(s)                       # tied group scores
    sigma = s.max(axis=0)
    for dstar in (0.0, 0.01, 0.1, 0.3, 0.9, 1.0):
        k = sdref.mass_budget_count(s, sigma, dstar, n)
        worst = lambda kk: max(sdref.dropped_mass(s[h], sdref.select_topk(sigma, kk)[0])
                               for h in range(G))
        assert worst(k) <= dstar + 1e-12 or k == n
        if k > 1:
            assert worst(k - 1) > dstar - 1e-12


def test_budget_edges_and_cap():
    rng = np.random.default_rng(5)
    s = rng.standard_normal((4, 300))
    sigma = s.max(axis=0)
    assert sdref.mass_budget_count(s, sigma, 1.0, 300) == 1
    assert sdref.mass_budget_count(s, sigma, 0.0, 300) == 300
    ks = [sdref.mass_budget_count(s, sigma, d, 300) for d in (0.001, 0.01, 0.05, 0.2, 0.5)]
    assert ks == sorted(ks, reverse=True)
    assert sdref.mass_budget_count(s, sigma, 0.001, 40) == 40          # the cap
    with pytest.raises(ValueError):
        sdref.mass_budget_count(s, sigma, -0.1, 300)


def test_budget_decode_step_reports_delta_within_target():
    w = kvsynth.generate(kvsynth.RECIPES["sweep"].with_(seq_len=2000, num_q_heads=8,
                                                         num_kv_heads=2))
    for dstar in (0.02, 0.1):
        sel = Sel("mass_budget", 0.5, max_dropped=dstar)
        res = sdref.decode_step(w.q, w.K, w.V, w.seq_lens, dtype="bf16", unit="token",
                                page_size=16, r_kv=0.5, selection=sel)
        for gr in res.values():
            cap = sdref.keep_count(0.5, 2000)
            assert 1 <= len(gr.kept) <= cap
            if len(gr.kept) < cap:
                assert gr.delta.max() <= dstar + 1e-12
    with pytest.raises(ValueError):
        sdref.decode_step(w.q, w.K, w.V, w.seq_lens, dtype="bf16", unit="page", page_size=16,
                          r_kv=0.5, selection=Sel("mass_budget", 0.5, max_dropped=0.1))
