"""Pins of the oracle's logits, attention, dropped mass and page bounds.

Each test checks the oracle against something other than itself: a worked
example with a hand-computed answer, a closed form, an identity that uses a
different route (attention over the complement), or a bound the mathematics
fixes.  Together they fail for a dropped scale, a wrong head-to-KV-head map,
a transposed operand, a missing renormalisation, a wrong sign in the page
bound, or bounds taken over invalid rows.
"""

import math

import numpy as np
import pytest

from oracle import sdref


# ---------------------------------------------------------------- logits

def test_logits_worked_example():
    # d = 4, scale 1/sqrt(4) = 1/2; q = (1, 2, 3, 4)
    q = np.array([[1.0, 2.0, 3.0, 4.0]])
    K = np.array([[[1.0, 0, 0, 0], [0, 0, 0, 1.0], [1.0, 1.0, 1.0, 1.0], [0, -1.0, 0, 0]]])
    s = sdref.logits(q, K, 0.5)
    assert s.shape == (1, 4)
    np.testing.assert_array_equal(s[0], [0.5, 2.0, 5.0, -1.0])


def test_logits_head_to_kv_head_map():
    """H_q = 4, H_kv = 2: heads 0, 1 read KV head 0 and heads 2, 3 read KV head 1."""
    q = np.arange(1, 4 * 3 + 1, dtype=float).reshape(4, 3)
    K = np.zeros((2, 2, 3))
    K[0, 0] = [1, 0, 0]       # KV head 0 picks channel 0
    K[1, 0] = [0, 0, 1]       # KV head 1 picks channel 2
    s = sdref.logits(q, K, 1.0)
    np.testing.assert_array_equal(s[:, 0], [q[0, 0], q[1, 0], q[2, 2], q[3, 2]])
    np.testing.assert_array_equal(s[:, 1], 0.0)
    np.testing.assert_array_equal(sdref.group_logits(q[2:4], K[1], 1.0), s[2:4])


# ---------------------------------------------------------------- attention

def test_attention_single_token():
    V = np.array([[3.0, -1.5, 2.0]])
    o, lse = sdref.attention(np.array([0.7]), V)
    np.testing.assert_array_equal(o, V[0])
    assert lse == 0.7


def test_attention_equal_logits_is_mean():
    rng = np.random.default_rng(0)
    V = rng.standard_normal((9, 5))
    o, lse = sdref.attention(np.full(9, -2.5), V)
    np.testing.assert_allclose(o, V.mean(axis=0), rtol=0, atol=1e-15)
    assert abs(lse - (-2.5 + math.log(9))) < 1e-15


def test_attention_worked_example_rational_weights():
    # weights proportional to 1, 2, 3 -> p = 1/6, 2/6, 3/6
    s = np.log(np.array([1.0, 2.0, 3.0])) + 4.0
    V = np.array([[6.0, 0.0], [0.0, 6.0], [1.0, 1.0]])
    o, lse = sdref.attention(s, V)
    np.testing.assert_allclose(o, [1.5, 2.5], rtol=0, atol=1e-14)
    assert abs(lse - (4.0 + math.log(6.0))) < 1e-14


def test_attention_two_tokens_is_logistic():
    # p_0 = 1 / (1 + e^{s1 - s0})
    s = np.array([1.3, -0.4])
    V = np.array([[1.0], [0.0]])
    o, _ = sdref.attention(s, V)
    assert abs(o[0] - 1.0 / (1.0 + math.exp(-1.7))) < 1e-15


def test_attention_shift_invariance_and_large_logits():
    rng = np.random.default_rng(1)
    s = rng.standard_normal(50) * 3
    V = rng.standard_normal((50, 4))
    o1, l1 = sdref.attention(s, V)
    o2, l2 = sdref.attention(s + 700.0, V)   # would overflow exp without the max shift
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
    assert abs((l2 - l1) - 700.0) < 1e-9


def test_attention_subset_matches_attention_on_sliced_arrays():
    rng = np.random.default_rng(2)
    s = rng.standard_normal(40)
    V = rng.standard_normal((40, 3))
    T = np.array([1, 5, 6, 30, 39])
    o1, l1 = sdref.attention(s, V, T)
    o2, l2 = sdref.attention(s[T].copy(), V[T].copy())
    np.testing.assert_array_equal(o1, o2)
    assert l1 == l2


# ---------------------------------------------------------------- split-K merge

def test_merge_worked_example():
    """Two one-token splits, s = (0, ln 3), V = (4, 0): the dense weights are
    1/4 and 3/4, so o = 1 and lse = ln 4 (by hand).  A merge that averaged the
    split outputs without their exp(lse) weights would give 2."""
    V = np.array([[4.0], [0.0]])
    s = np.array([0.0, math.log(3.0)])
    o, lse = sdref.split_attention(s, V, [np.array([0]), np.array([1])])
    np.testing.assert_allclose(o, [1.0], rtol=0, atol=1e-15)
    assert abs(lse - math.log(4.0)) < 1e-15


@pytest.mark.parametrize("seed", range(6))
def test_merge_partition_invariance_with_empty_splits(seed):
    """Any partition of the attended tokens into splits, empty ones included
    and in any order, merges to the one-shot attention over their union
    (to fp64 rounding: 1e-13)."""
    rng = np.random.default_rng(100 + seed)
    n, d = int(rng.integers(1, 400)), 16
    s = rng.standard_normal(n) * 4.0
    V = rng.standard_normal((n, d))
    tokens = np.sort(rng.choice(n, size=int(rng.integers(1, n + 1)), replace=False))
    o1, l1 = sdref.attention(s, V, tokens)
    for _ in range(5):
        S = int(rng.integers(1, 40))
        owner = rng.integers(0, S, size=tokens.size)          # random split of each token
        splits = [tokens[owner == j] for j in range(S)]       # many are empty when S > |T|
        splits += [np.array([], dtype=np.int64)] * int(rng.integers(0, 3))
        rng.shuffle(splits)
        o2, l2 = sdref.split_attention(s, V, splits)
        np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-13)
        assert abs(l2 - l1) < 1e-13


def test_merge_contiguous_splits_of_the_dense_row():
    """Contiguous equal splits, as a split-K kernel cuts a kept list, with a
    trailing empty split: the dense result."""
    rng = np.random.default_rng(7)
    n = 1000
    s = rng.standard_normal(n) * 3.0
    V = rng.standard_normal((n, 8))
    E = 96
    splits = [np.arange(j * E, min((j + 1) * E, n)) for j in range(-(-n // E) + 1)]
    assert splits[-1].size == 0
    o, lse = sdref.split_attention(s, V, splits)
    o1, l1 = sdref.attention(s, V)
    np.testing.assert_allclose(o, o1, rtol=0, atol=1e-13)
    assert abs(lse - l1) < 1e-13


def test_merge_empty_and_single_split():
    V = np.arange(6.0).reshape(3, 2)
    s = np.array([0.5, -1.0, 2.0])
    o, lse = sdref.merge_splits([sdref.split_partial(s, V, [])] * 3)
    np.testing.assert_array_equal(o, [0.0, 0.0])
    assert lse == -math.inf
    only = sdref.split_partial(s, V, [0, 2])
    o, lse = sdref.merge_splits([sdref.split_partial(s, V, []), only, sdref.split_partial(s, V, [])])
    np.testing.assert_array_equal(o, only[0])
    assert lse == only[1]


# ---------------------------------------------------------------- dropped mass

def test_dropped_mass_worked_example():
    s = np.log(np.array([1.0, 2.0, 3.0, 4.0]))     # p = 0.1, 0.2, 0.3, 0.4
    assert abs(sdref.dropped_mass(s, np.array([1, 3])) - 0.4) < 1e-15
    assert sdref.dropped_mass(s, np.arange(4)) == 0.0


@pytest.mark.parametrize("seed", range(20))
def test_sparse_dense_decomposition_and_error_bound(seed):
    """o = (1 - delta) o_T + delta o_D, with o_D the attention over the dropped
    set; lse_T = lse + log(1 - delta); and |o - o_T| <= 2 delta max|V| in the
    2-norm and the max-norm."""
    rng = np.random.default_rng(seed)
    n, d = int(rng.integers(2, 200)), 8
    s = rng.standard_normal(n) * rng.uniform(0.1, 4)
    V = rng.standard_normal((n, d)) * rng.uniform(0.1, 3)
    m = int(rng.integers(1, n))
    T = np.sort(rng.choice(n, size=m, replace=False))
    D = np.setdiff1d(np.arange(n), T)
    o, lse = sdref.attention(s, V)
    oT, lT = sdref.attention(s, V, T)
    oD, _ = sdref.attention(s, V, D)
    delta = sdref.dropped_mass(s, T)
    assert 0.0 < delta < 1.0
    np.testing.assert_allclose(o, (1 - delta) * oT + delta * oD, rtol=0, atol=1e-12)
    assert abs(lT - (lse + math.log1p(-delta))) < 1e-12
    vmax2 = np.linalg.norm(V, axis=1).max()
    vmaxinf = np.abs(V).max()
    assert np.linalg.norm(o - oT) <= 2 * delta * vmax2 + 1e-12
    assert np.abs(o - oT).max() <= 2 * delta * vmaxinf + 1e-12


# ---------------------------------------------------------------- page bounds

def test_page_bounds_valid_rows_only():
    K = np.arange(17 * 2, dtype=float).reshape(17, 2)
    kmin, kmax = sdref.page_bounds(K, 16)
    assert kmin.shape == (2, 2)
    np.testing.assert_array_equal(kmin[0], K[0])
    np.testing.assert_array_equal(kmax[0], K[15])
    np.testing.assert_array_equal(kmin[1], K[16])
    np.testing.assert_array_equal(kmax[1], K[16])


def test_page_score_worked_example():
    # q = (1, -1); page rows (1, 2) and (3, -4): kmin = (1, -4), kmax = (3, 2)
    # sum_c max(q_c kmin_c, q_c kmax_c) = max(1, 3) + max(4, -2) = 7
    K = np.array([[1.0, 2.0], [3.0, -4.0]])
    kmin, kmax = sdref.page_bounds(K, 2)
    sig = sdref.page_scores(np.array([[1.0, -1.0]]), kmin, kmax, 0.5)
    assert sig.shape == (1,)
    assert sig[0] == 3.5
    # the group maximum: a second head (0, 1) scores max(-4, 2) * 0.5 = 1, below 3.5
    sig2 = sdref.page_scores(np.array([[0.0, 1.0], [1.0, -1.0]]), kmin, kmax, 0.5)
    assert sig2[0] == 3.5


@pytest.mark.parametrize("seed", range(10))
def test_page_score_bounds_every_token_logit(seed):
    rng = np.random.default_rng(100 + seed)
    G, n, d, P = 4, int(rng.integers(1, 300)), 16, int(rng.choice([1, 4, 16, 64]))
    q = rng.standard_normal((G, d))
    K = rng.standard_normal((n, d)) * rng.uniform(0.5, 2, size=d)
    scale = 1 / math.sqrt(d)
    kmin, kmax = sdref.page_bounds(K, P)
    sig = sdref.page_scores(q, kmin, kmax, scale)
    s = sdref.group_logits(q, K, scale)
    for u in range(sig.shape[0]):
        page_max = s[:, u * P:min((u + 1) * P, n)].max()
        assert sig[u] >= page_max - 1e-12


def test_page_unit_of_one_token_is_token_unit():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((3, 8))
    K = rng.standard_normal((25, 8))
    kmin, kmax = sdref.page_bounds(K, 1)
    np.testing.assert_array_equal(kmin, K)
    np.testing.assert_array_equal(kmax, K)
    sig_page = sdref.page_scores(q, kmin, kmax, 0.25)
    sig_tok = sdref.token_scores(sdref.group_logits(q, K, 0.25))
    np.testing.assert_allclose(sig_page, sig_tok, rtol=0, atol=1e-13)


def test_token_scores_group_max():
    s = np.array([[1.0, -2.0, 0.5], [0.0, 3.0, 0.25]])
    np.testing.assert_array_equal(sdref.token_scores(s), [1.0, 3.0, 0.5])


def test_widen_bf16_and_f32():
    bits = np.array([0x3F80, 0xC040, 0x0000, 0x8000, 0x3F81], dtype=np.uint16)
    np.testing.assert_array_equal(sdref.widen(bits, "bf16"), [1.0, -3.0, 0.0, -0.0, 1.0 + 2.0 ** -7])
    x = np.array([0.1, -2.5], dtype=np.float32)
    np.testing.assert_array_equal(sdref.widen(x, "f32"), x.astype(np.float64))
