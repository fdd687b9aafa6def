"""Pins of the oracle's keep count, top-k selection and whole decode step.

* keep count: the configurations' stated counts, and the exact decimal
  ceiling ceil(r * U) computed with fractions from the decimal text of r;
* selection: an O(n^2) rank count over n <= 64 (random and tied scores), and
  exhaustive subsets for n <= 12 showing the top-k set drops the least mass;
* decode step: a keep ratio of 1 gives dense attention exactly with zero
  dropped mass; outputs obey the 2 * delta * max|V| bound; a page of one
  token is the token unit.
"""

import itertools
import math
from fractions import Fraction

import numpy as np
import pytest

import kvsynth
from oracle import sdref


# ---------------------------------------------------------------- keep count

@pytest.mark.parametrize("r,U,k", [
    (0.25, 1024, 256),     # tiny config: 256 tokens
    (0.3, 2048, 615),      # 8B-shaped page config: 614.4 -> 615
    (0.05, 2048, 103),     # 70B-shaped at 128K, page 64
    (0.05, 16384, 820),    # 70B-shaped at 1M, page 64
    (0.3, 131072, 39322),
    (0.2, 131072, 26215),
    (0.07, 100, 7),        # 0.07 * 100 is 7.000000000000001 in binary floating point
    (1.0, 77, 77),
    (3.0, 5, 5),
    (1e-9, 1000, 1),
    (0.9999999, 10, 10),
])
def test_keep_count_values(r, U, k):
    assert sdref.keep_count(r, U) == k


@pytest.mark.parametrize("seed", range(5))
def test_keep_count_is_decimal_ceiling(seed):
    rng = np.random.default_rng(seed)
    for _ in range(400):
        r = round(float(rng.uniform(1e-6, 1.0)), int(rng.integers(1, 7)))
        if r <= 0:
            continue
        U = int(rng.integers(1, 300000))
        exact = math.ceil(Fraction(repr(r)) * U)
        assert sdref.keep_count(r, U) == min(max(exact, 1), U)


@pytest.mark.parametrize("r", [0.0, -0.5, float("nan"), float("inf")])
def test_keep_count_rejects(r):
    with pytest.raises(ValueError):
        sdref.keep_count(r, 10)


# ---------------------------------------------------------------- top-k

def _rank_count_set(sigma, k):
    n = len(sigma)
    keep = []
    for u in range(n):
        ahead = sum(1 for v in range(n) if sigma[v] > sigma[u] or (sigma[v] == sigma[u] and v < u))
        if ahead < k:
            keep.append(u)
    return np.array(keep, dtype=np.int64)


@pytest.mark.parametrize("seed", range(30))
def test_topk_matches_rank_count(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 65))
    if seed % 3 == 0:
        sigma = rng.integers(-3, 4, size=n).astype(float)       # many ties
    elif seed % 3 == 1:
        sigma = rng.standard_normal(n)
    else:
        sigma = np.round(rng.standard_normal(n), 1) * 0.0 + rng.choice([-0.0, 0.0, 1.0], size=n)
    for k in range(1, n + 1):
        kept, gap = sdref.select_topk(sigma, k)
        np.testing.assert_array_equal(kept, _rank_count_set(sigma, k))
        assert np.all(np.diff(kept) > 0)
        if k < n:
            dropped = np.setdiff1d(np.arange(n), kept)
            assert gap == sigma[kept].min() - sigma[dropped].max()
        else:
            assert gap == math.inf


def test_topk_ties_go_to_lower_index():
    sigma = np.array([1.0, 5.0, 5.0, 2.0, 5.0, 5.0])
    kept, gap = sdref.select_topk(sigma, 3)
    np.testing.assert_array_equal(kept, [1, 2, 4])
    assert gap == 0.0
    kept, _ = sdref.select_topk(np.array([0.0, -0.0, 0.0]), 2)   # -0 and +0 tie
    np.testing.assert_array_equal(kept, [0, 1])


@pytest.mark.parametrize("seed", range(12))
def test_topk_minimises_dropped_mass(seed):
    """Token unit, one query head: keeping the k largest logits drops the
    least softmax mass among all C(n, k) subsets."""
    rng = np.random.default_rng(seed)
    n = int(rng.integers(2, 13))
    q = rng.standard_normal((1, 4))
    K = rng.standard_normal((n, 4))
    s = sdref.group_logits(q, K, 0.5)
    sigma = sdref.token_scores(s)
    for k in range(1, n):
        kept, _ = sdref.select_topk(sigma, k)
        best = sdref.dropped_mass(s[0], kept)
        for subset in itertools.combinations(range(n), k):
            assert best <= sdref.dropped_mass(s[0], np.array(subset)) + 1e-15


# ---------------------------------------------------------------- decode step

def _small(recipe, n):
    return kvsynth.generate(recipe.with_(seq_len=n))


@pytest.mark.parametrize("unit,P", [("token", 16), ("page", 16), ("page", 64)])
def test_keep_ratio_one_is_dense(unit, P):
    w = _small(kvsynth.RECIPES["l8b"].with_(unit=unit, page_size=P, num_q_heads=8, num_kv_heads=2), 1000)
    res = sdref.decode_step(w.q, w.K, w.V, w.seq_lens, dtype="bf16", unit=unit, page_size=P, r_kv=1.0)
    for g in res.values():
        np.testing.assert_array_equal(g.out_sparse, g.out_dense)
        np.testing.assert_array_equal(g.lse_sparse, g.lse_dense)
        assert np.all(g.delta == 0.0)


@pytest.mark.parametrize("name,n,unit,P,r", [
    ("tiny", 1024, "token", 16, 0.25),
    ("l8b", 3000, "page", 16, 0.3),
    ("l70b", 5000, "page", 64, 0.05),
    ("sweep", 2048, "token", 16, 0.2),
])
def test_config_shaped_steps_obey_delta_bound(name, n, unit, P, r):
    rec = kvsynth.RECIPES[name].with_(seq_len=n, unit=unit, page_size=P, r_kv=r)
    w = kvsynth.generate(rec)
    res = sdref.decode_step(w.q, w.K, w.V, w.seq_lens, dtype=rec.dtype, unit=unit,
                            page_size=P, r_kv=r)
    G = rec.group
    for (b, g), gr in res.items():
        V = sdref.widen(w.V[b, g, :n], rec.dtype)
        vmax = np.linalg.norm(V, axis=1).max()
        U = sdref.num_units(n, unit, P)
        assert gr.k == sdref.keep_count(r, U) and len(gr.kept) == gr.k
        for i in range(G):
            err = np.linalg.norm(gr.out_sparse[i] - gr.out_dense[i])
            assert err <= 2 * gr.delta[i] * vmax + 1e-12
            assert 0.0 <= gr.delta[i] < 1.0


def test_page_of_one_token_equals_token_unit():
    rec = kvsynth.RECIPES["l8b"].with_(seq_len=300, num_q_heads=8, num_kv_heads=2)
    w = kvsynth.generate(rec)
    tok = sdref.decode_step(w.q, w.K, w.V, w.seq_lens, dtype="bf16", unit="token", page_size=1, r_kv=0.3)
    pag = sdref.decode_step(w.q, w.K, w.V, w.seq_lens, dtype="bf16", unit="page", page_size=1, r_kv=0.3)
    for key in tok:
        a, b = tok[key], pag[key]
        np.testing.assert_allclose(a.sigma, b.sigma, rtol=0, atol=1e-12)
        if a.gap > 1e-9:
            np.testing.assert_array_equal(a.kept, b.kept)
            np.testing.assert_allclose(a.out_sparse, b.out_sparse, rtol=0, atol=1e-13)


def test_tiny_salient_keys_dominate_selection():
    """In the tiny configuration the planted keys sit about 3|q|/8 logits above
    the rest, so nearly all of them are kept; the dropped mass stays well above
    zero because 1024 ordinary keys carry a heavy softmax tail (how much
    depends on each query's norm: a longer query concentrates more mass on its
    planted keys)."""
    w = kvsynth.generate(kvsynth.RECIPES["tiny"])
    res = sdref.decode_step(w.q, w.K, w.V, w.seq_lens, dtype="f32", unit="token", page_size=16, r_kv=0.25)
    gr = res[(0, 0)]
    planted = w.salient[(0, 0)]
    assert planted.size == 128
    assert np.isin(planted, gr.kept).mean() > 0.9
    assert np.all((gr.delta > 0.02) & (gr.delta < 0.8))
    assert gr.delta.mean() > 0.15
