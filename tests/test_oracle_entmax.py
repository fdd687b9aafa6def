"""Pins of the alpha-entmax oracle (oracle/entmaxref.py).

[Cross/cards], EntmaxKV abstract: alpha-entmax has exact zeros, sparse
decoding is exact once the kept candidates hold the support, and the output
error is governed by the dropped mass delta.  The map is pinned against
things other than its own bisection:
* the variational definition (argmax over the simplex of p.z plus the Tsallis
  entropy), solved by a generic constrained optimiser;
* the sort-based closed forms of sparsemax (alpha = 2) and of 1.5-entmax
  (for a support of size k the threshold solves a quadratic);
* the softmax limit alpha -> 1 with an error linear in alpha - 1;
* closed-form special cases (one logit, ties, a gap of 1 / (alpha - 1));
* support recovery (exact output, delta = 0) and the 2 delta max|v| bound.
"""

import math

import numpy as np
import pytest
from scipy.optimize import minimize

from oracle import entmaxref as E
from oracle import sdref


def _sparsemax_sorted(z):
    """Sparsemax by sorting: the support size is the largest k with
    1 + k z_(k) > sum_{j <= k} z_(j), and tau = (sum_{j <= k} z_(j) - 1) / k."""
    zs = np.sort(np.asarray(z, np.float64))[::-1]
    cs = np.cumsum(zs)
    ks = np.arange(1, zs.size + 1)
    k = int(ks[1.0 + ks * zs > cs].max())
    tau = (cs[k - 1] - 1.0) / k
    return np.maximum(z - tau, 0.0), tau


def _entmax15_sorted(z):
    """1.5-entmax by sorting.  With x = z / 2 and support size k, the threshold
    solves sum_{i <= k} (x_(i) - tau)^2 = 1; the smaller root is
    tau_k = mu_k - sqrt(1/k - (msq_k - mu_k^2)) (mu, msq: the mean and the mean
    square of the k largest x).  The support is the largest k whose root
    stays below x_(k)."""
    x = np.asarray(z, np.float64) / 2.0
    xs = np.sort(x)[::-1]
    best = None
    for k in range(1, xs.size + 1):
        mu = xs[:k].mean()
        msq = (xs[:k] ** 2).mean()
        disc = 1.0 / k - (msq - mu * mu)
        if disc < 0:
            break
        tau = mu - math.sqrt(disc)
        if tau < xs[k - 1]:
            best = tau
    return np.maximum(x - best, 0.0) ** 2, best


def _tsallis_argmax(z, alpha):
    """argmax over the simplex of p.z + (1 - sum p^alpha) / (alpha (alpha - 1)),
    by SLSQP from the uniform point (the definition of alpha-entmax)."""
    z = np.asarray(z, np.float64)
    n = z.size

    def neg(p):
        p = np.maximum(p, 0.0)
        return -(p @ z + (1.0 - np.sum(p ** alpha)) / (alpha * (alpha - 1.0)))

    res = minimize(neg, np.full(n, 1.0 / n), method="SLSQP", bounds=[(0.0, 1.0)] * n,
                   constraints=[{"type": "eq", "fun": lambda p: p.sum() - 1.0}],
                   options={"ftol": 1e-15, "maxiter": 1000})
    return np.maximum(res.x, 0.0)


@pytest.mark.parametrize("alpha", [1.25, 1.5, 1.75, 2.0])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_variational_definition(alpha, seed):
    z = np.random.default_rng(seed).normal(size=7) * 1.5
    p, _ = E.entmax(z, alpha)
    ref = _tsallis_argmax(z, alpha)
    assert np.abs(p - ref).max() < 2e-5


@pytest.mark.parametrize("seed", range(6))
def test_sparsemax_closed_form(seed):
    z = np.random.default_rng(seed).normal(size=40) * 0.7
    p, tau = E.entmax(z, 2.0)
    ref, tau_ref = _sparsemax_sorted(z)
    assert abs(tau - tau_ref) < 1e-13
    assert np.abs(p - ref).max() < 1e-13


@pytest.mark.parametrize("seed", range(6))
def test_entmax15_closed_form(seed):
    z = np.random.default_rng(seed + 10).normal(size=60) * 2.0
    p, tau = E.entmax(z, 1.5)
    ref, tau_ref = _entmax15_sorted(z)
    assert abs(tau - tau_ref) < 1e-13
    assert np.abs(p - ref).max() < 1e-13


def test_softmax_limit():
    z = np.random.default_rng(3).normal(size=50) * 2.0
    w = np.exp(z - z.max())
    soft = w / w.sum()
    errs = [np.abs(E.entmax(z, 1.0 + eps)[0] - soft).max() for eps in (1e-2, 1e-3, 1e-4)]
    assert errs[2] < 5e-4
    # first order in alpha - 1: each tenfold step shrinks the error about tenfold
    assert 7.0 < errs[0] / errs[1] < 13.0 and 7.0 < errs[1] / errs[2] < 13.0


@pytest.mark.parametrize("alpha", [1.25, 1.5, 2.0])
def test_special_cases(alpha):
    # one logit
    p, _ = E.entmax(np.array([0.3]), alpha)
    assert p.tolist() == [1.0]
    # equal logits: uniform
    p, _ = E.entmax(np.full(5, -1.7), alpha)
    assert np.abs(p - 0.2).max() < 1e-14
    # a lead of 1 / (alpha - 1) over the rest: one-hot (the top term alone is 1
    # at tau = x_max - 1, where every other term is 0)
    z = np.array([0.0, -1.0 / (alpha - 1.0), -5.0])
    p, _ = E.entmax(z, alpha)
    assert p.tolist() == [1.0, 0.0, 0.0]
    # shift invariance and permutation equivariance
    z = np.random.default_rng(5).normal(size=20)
    p, _ = E.entmax(z, alpha)
    assert np.abs(E.entmax(z + 3.25, alpha)[0] - p).max() < 1e-12
    perm = np.random.default_rng(6).permutation(20)
    assert np.abs(E.entmax(z[perm], alpha)[0] - p[perm]).max() < 1e-12


def test_rejects_bad_input():
    for bad in (1.0, 0.5, 2.5, float("nan")):
        with pytest.raises(ValueError):
            E.entmax(np.zeros(3), bad)
    with pytest.raises(ValueError):
        E.entmax(np.array([0.0, np.inf]), 1.5)
    with pytest.raises(ValueError):
        E.entmax(np.zeros(0), 1.5)


@pytest.mark.parametrize("alpha", [1.25, 1.5, 2.0])
def test_support_recovery_is_exact(alpha):
    rng = np.random.default_rng(11)
    n, d = 300, 16
    s = rng.normal(size=n) * 3.0
    V = rng.normal(size=(n, d))
    p, _ = E.entmax(s, alpha)
    supp = np.flatnonzero(p > 0)
    assert supp.size < n // 2
    o, _, _ = E.entmax_attention(s, V, alpha)
    extra = rng.choice(np.setdiff1d(np.arange(n), supp), size=40, replace=False)
    tokens = np.sort(np.concatenate([supp, extra]))
    o_s, _, _ = E.entmax_attention(s, V, alpha, tokens)
    assert E.entmax_dropped_mass(s, tokens, alpha) == 0.0
    assert np.abs(o - o_s).max() < 1e-12


@pytest.mark.parametrize("alpha", [1.25, 1.5, 2.0])
@pytest.mark.parametrize("seed", range(4))
def test_dropped_mass_bounds_the_error(alpha, seed):
    """With T missing part of the support, tau over T is lower, every kept
    weight grows (p'_t >= p_t on T) and the growth sums to delta, so
    |o - o_S| <= delta max|v| + delta max|v|."""
    rng = np.random.default_rng(seed + 20)
    n, d = 200, 8
    s = rng.normal(size=n) * 2.0
    V = rng.normal(size=(n, d))
    p, _ = E.entmax(s, alpha)
    supp = np.flatnonzero(p > 0)
    drop = rng.choice(supp, size=max(1, supp.size // 3), replace=False)
    tokens = np.setdiff1d(np.arange(n), drop)
    delta = E.entmax_dropped_mass(s, tokens, alpha)
    assert delta > 0
    p_t, _ = E.entmax(s[tokens], alpha)
    assert np.all(p_t >= p[tokens] - 1e-15)
    assert abs((p_t - p[tokens]).sum() - delta) < 1e-12
    o, _, _ = E.entmax_attention(s, V, alpha)
    o_s, _, _ = E.entmax_attention(s, V, alpha, tokens)
    vmax = np.linalg.norm(V, axis=1).max()
    assert np.linalg.norm(o - o_s) <= 2 * delta * vmax + 1e-12


def test_group_step_full_keep_is_dense():
    rng = np.random.default_rng(4)
    G, n, d = 4, 100, 16
    q = rng.normal(size=(G, d)); K = rng.normal(size=(n, d)); V = rng.normal(size=(n, d))
    for unit in ("token", "page"):
        r = E.group_step(q, K, V, unit=unit, page_size=16, r_kv=1.0, scale=0.25)
        assert np.abs(r.out_sparse - r.out_dense).max() < 1e-13
        assert np.all(r.delta == 0.0)
        assert np.abs(r.tau_sparse - r.tau_dense).max() < 1e-13


def test_group_step_selection_is_the_softmax_paths():
    rng = np.random.default_rng(8)
    G, n, d = 2, 333, 16
    q = rng.normal(size=(G, d)); K = rng.normal(size=(n, d)); V = rng.normal(size=(n, d))
    for unit in ("token", "page"):
        a = E.group_step(q, K, V, unit=unit, page_size=16, r_kv=0.3, scale=0.25)
        b = sdref.group_step(q, K, V, unit=unit, page_size=16, r_kv=0.3, scale=0.25)
        assert np.array_equal(a.kept, b.kept) and a.k == b.k
        tokens = sdref.unit_tokens(a.kept, unit, 16, n)
        s = sdref.group_logits(q, K, 0.25)
        for i in range(G):
            o, tau, _ = E.entmax_attention(s[i], V, 1.5, tokens)
            assert np.abs(o - a.out_sparse[i]).max() < 1e-14 and tau == a.tau_sparse[i]


def test_needles_are_recovered():
    """On the tiny needle inputs, 1.5-entmax puts its support on few keys and
    token top-k at r = 0.25 holds all of it: the sparse output is exact."""
    import kvsynth
    rec = kvsynth.RECIPES["tiny"]
    w = kvsynth.generate(rec)
    n = int(w.seq_lens[0])
    q = sdref.widen(w.q[0], rec.dtype)
    K = sdref.widen(w.K[0, 0, :n], rec.dtype)
    V = sdref.widen(w.V[0, 0, :n], rec.dtype)
    r = E.group_step(q, K, V, unit="token", page_size=rec.page_size, r_kv=rec.r_kv,
                     scale=1.0 / math.sqrt(rec.head_dim))
    assert np.all(r.support < r.k)
    assert np.all(r.delta == 0.0)
    assert np.abs(r.out_sparse - r.out_dense).max() < 1e-12
