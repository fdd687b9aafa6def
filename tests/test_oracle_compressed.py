"""Pins of the oracle's compressed-key page scorer.

* windowing: every token lies in two windows (one for the first 16), so the
  count-weighted window means sum to the tokens' keys weighted that way;
* constant keys give equal scores (the top-k is then the first pages);
* a single non-zero key lifts exactly the pages holding the starts of the two
  windows that cover it, with the closed-form value;
* scores scale linearly with the keys and the summed queries;
* the number of scored pages is the page count for ragged lengths at pages
  of 16 and 64 tokens (the pages' 64-token blocks pool four windows);
* on the planted-page inputs the compressed keys find every planted page
  and the page bound misses them (its per-channel extremes over 64 ordinary
  keys are wider than a planted page's).
"""

import numpy as np
import pytest

import kvsynth
from oracle import sdref


@pytest.mark.parametrize("n", [1, 15, 16, 17, 31, 32, 33, 100, 640, 1001])
def test_windows_cover_every_token_twice(n):
    rng = np.random.default_rng(n)
    K = rng.standard_normal((n, 8))
    c = sdref.compressed_keys(K)
    J = c.shape[0]
    assert J == -(-n // 16)
    counts = np.array([min(16 * j + 32, n) - 16 * j for j in range(J)])
    weights = np.where(np.arange(n) < 16, 1.0, 2.0)
    np.testing.assert_allclose((c * counts[:, None]).sum(axis=0), (K * weights[:, None]).sum(axis=0),
                               rtol=0, atol=1e-12)


def test_constant_keys_tie_every_page():
    v = np.linspace(-1, 1, 8)
    K = np.tile(v, (700, 1))
    q = np.random.default_rng(1).standard_normal((4, 8))
    for P in (16, 64):
        s = sdref.compressed_page_scores(q, sdref.compressed_keys(K), P, 0.5)
        np.testing.assert_allclose(s, 0.5 * q.sum(axis=0) @ v, rtol=0, atol=1e-12)
        kept, _ = sdref.select_topk(s, 3)
        np.testing.assert_array_equal(kept, [0, 1, 2])


@pytest.mark.parametrize("t", [0, 5, 16, 40, 63, 64, 100, 639])
@pytest.mark.parametrize("P", [16, 64])
def test_single_key_lifts_the_pages_of_its_windows(t, P):
    n, d = 640, 8
    K = np.zeros((n, d))
    K[t, 3] = 1.0
    q = np.zeros((2, d))
    q[:, 3] = [0.7, 0.5]                       # summed query 1.2 on channel 3
    s = sdref.compressed_page_scores(q, sdref.compressed_keys(K), P, 2.0)
    windows = [j for j in (t // 16 - 1, t // 16) if j >= 0]
    lifted = sorted({(16 * j) // P for j in windows})
    expect = np.zeros(len(s))
    for j in windows:
        cnt = min(16 * j + 32, n) - 16 * j
        expect[(16 * j) // P] = max(expect[(16 * j) // P], 2.0 * 1.2 / cnt)
    np.testing.assert_allclose(s, expect, rtol=0, atol=1e-15)
    assert sorted(np.flatnonzero(s > 0).tolist()) == lifted


def test_scores_are_linear():
    rng = np.random.default_rng(3)
    K = rng.standard_normal((300, 16))
    q = rng.standard_normal((4, 16))
    base = sdref.compressed_page_scores(q, sdref.compressed_keys(K), 64, 0.25)
    scaled = sdref.compressed_page_scores(q, sdref.compressed_keys(3.0 * K), 64, 0.25)
    np.testing.assert_allclose(scaled, 3.0 * base, rtol=1e-12, atol=0)
    # summing the relevance over heads is the relevance of the summed query
    one = sdref.compressed_page_scores(q.sum(axis=0, keepdims=True), sdref.compressed_keys(K),
                                       64, 0.25)
    np.testing.assert_allclose(one, base, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("P", [16, 64])
def test_page_count_and_decode_step(P):
    rec = kvsynth.RECIPES["batch"].with_(batch=3, seq_len=2000, seq_len_min=1, page_size=P,
                                         num_q_heads=8, num_kv_heads=2)
    w = kvsynth.generate(rec)
    res = sdref.decode_step(w.q, w.K, w.V, w.seq_lens, dtype="bf16", unit="page", page_size=P,
                            r_kv=0.2, scorer="compressed")
    for (b, g), gr in res.items():
        n = int(w.seq_lens[b])
        assert gr.sigma.shape[0] == sdref.num_units(n, "page", P)
        assert len(gr.kept) == sdref.keep_count(0.2, gr.sigma.shape[0])
        V = sdref.widen(w.V[b, g, :n], "bf16")
        vmax = np.linalg.norm(V, axis=1).max()
        for i in range(rec.group):
            assert np.linalg.norm(gr.out_sparse[i] - gr.out_dense[i]) <= 2 * gr.delta[i] * vmax + 1e-12


def test_recall_of_planted_pages_both_scorers():
    """The 70B-shaped inputs plant 1% salient pages (every token a salient
    key, 3 q_hat + N(0, 0.5^2)).  At r = 0.05 the compressed-key scorer keeps
    every planted page, while the page bound misses them: over 64 ordinary
    keys the per-channel extremes are wide, and the bound sum_c max(q kmin,
    q kmax) of an ordinary page exceeds that of a planted one.  The recall
    and dropped mass of both are printed (the comparison a second scorer is
    for)."""
    rec = kvsynth.RECIPES["l70b"].with_(seq_len=16384)
    w = kvsynth.generate(rec)
    groups = [(0, g) for g in range(rec.num_kv_heads)]
    res = {}
    for scorer in ("bounds", "compressed"):
        res[scorer] = sdref.decode_step(w.q, w.K, w.V, w.seq_lens, dtype="bf16", unit="page",
                                        page_size=64, r_kv=0.05, groups=groups, scorer=scorer)
    recall, delta = {}, {}
    for scorer, rr in res.items():
        recall[scorer] = np.mean([np.isin(w.salient_pages[k], rr[k].kept).mean() for k in groups])
        delta[scorer] = np.mean([rr[k].delta.mean() for k in groups])
        print(f"[recall] {scorer}: planted-page recall {recall[scorer]:.3f}, "
              f"mean delta {delta[scorer]:.4f}")
    assert recall["compressed"] == 1.0
    assert recall["bounds"] < 0.5
    assert delta["compressed"] < delta["bounds"]
