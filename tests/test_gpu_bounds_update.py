"""Row a0 as a decode loop runs it: page statistics kept current token by
token ("Where Activation Sparsity and KV-Cache Sparsity Cross in LLM
Decoding", cards view, EntmaxKV abstract: the page statistics are known
before any page is loaded, so they must follow every appended token).

A ragged batch grows across page boundaries; after every step only the
touched pages are updated -- by the O(d) append fold, or by recomputing the
listed (sequence, logical page) pairs -- and every valid page's bounds must
equal the oracle's min / max over its valid tokens bit for bit.
"""

import numpy as np
import pytest
import torch

import kvsynth
import sparse_kv_cache_sd_amd as sd
from oracle import sdref

from gpu_util import host_f64, upload

pytestmark = pytest.mark.gpu


def _check_all(dev, lens):
    s, w = dev.shape, dev.w
    got = host_f64(dev.bounds)
    for b in range(s.batch):
        n = int(lens[b])
        if n == 0:
            continue
        for g in range(s.num_kv_heads):
            kmin, kmax = sdref.page_bounds(sdref.widen(w.K[b, g, :n], s.dtype), s.page_size)
            U = kmin.shape[0]
            np.testing.assert_array_equal(got[b, g, :U, 0], kmin, err_msg=f"b={b} g={g} n={n}")
            np.testing.assert_array_equal(got[b, g, :U, 1], kmax, err_msg=f"b={b} g={g} n={n}")


# (recipe, overrides, per-step growth pattern)
CASES = [
    ("batch", dict(batch=4, seq_len=700, seq_len_min=600, num_q_heads=8, num_kv_heads=2), "append"),
    ("batch", dict(batch=4, seq_len=700, seq_len_min=600, num_q_heads=8, num_kv_heads=2), "list"),
    ("l70b", dict(batch=3, seq_len=64 * 6 + 9, num_q_heads=16, num_kv_heads=2), "append"),
    ("l70b", dict(batch=3, seq_len=64 * 6 + 9, num_q_heads=16, num_kv_heads=2), "list"),
    ("tiny", dict(batch=2, seq_len=300), "append"),
]


@pytest.mark.parametrize("name,kw,mode", CASES, ids=[f"{c[0]}-P{kvsynth.RECIPES[c[0]].page_size}-{c[2]}"
                                                      for c in CASES])
def test_bounds_follow_appended_tokens(name, kw, mode):
    rec = kvsynth.RECIPES[name].with_(**kw)
    w = kvsynth.generate(rec)
    dev = upload(w)                       # bounds of the final lengths; overwritten below
    s = dev.shape
    P = s.page_size
    final = w.seq_lens.astype(np.int64)
    rng = np.random.default_rng(11)
    # start short and ragged: empty, one token, mid-page and page-aligned lengths
    lens = np.array([[0, 1, P - 1, 2 * P][b % 4] for b in range(s.batch)], dtype=np.int64)
    lens = np.minimum(lens, final)
    dev.bounds.fill_(float("nan"))
    dev.sl.copy_(torch.from_numpy(lens.astype(np.int32)))
    sd.update_page_bounds(s, dev.k, dev.bt, dev.sl, dev.bounds)
    torch.cuda.synchronize()
    _check_all(dev, lens)
    steps = 0
    while np.any(lens < final):
        # mostly one token per step (a decode step); now and then a burst that
        # crosses one or more page boundaries (several tokens accepted at once)
        burst = rng.random(s.batch) < 0.15
        add = np.where(burst, rng.integers(2, 2 * P + 3, size=s.batch), 1)
        add = np.minimum(add, final - lens)
        new = lens + add
        dev.sl.copy_(torch.from_numpy(new.astype(np.int32)))
        if mode == "append":
            sd.append_page_bounds(s, dev.k, dev.bt, dev.sl,
                                  torch.from_numpy(add.astype(np.int32)).cuda(),
                                  int(max(1, add.max())), dev.bounds)
        else:
            pairs = [(b, u) for b in range(s.batch) if add[b] > 0
                     for u in range(int(lens[b]) // P, (int(new[b]) - 1) // P + 1)]
            pages = torch.tensor(pairs if pairs else [[0, 0]], dtype=torch.int32).reshape(-1, 2)
            sd.update_page_bounds(s, dev.k, dev.bt, dev.sl, dev.bounds,
                                  pages=pages[:len(pairs)].contiguous().cuda())
        lens = new
        steps += 1
        if steps % 7 == 0 or np.all(lens == final):
            torch.cuda.synchronize()
            _check_all(dev, lens)
    torch.cuda.synchronize()
    _check_all(dev, lens)
    print(f"[bounds] {name} P={P} {mode}: {steps} steps to lengths {final.tolist()}", flush=True)


def test_listed_pages_only():
    """Only the listed pairs are written; pairs past a sequence's end or
    outside the batch are skipped; an empty list writes nothing."""
    rec = kvsynth.RECIPES["batch"].with_(batch=3, seq_len=500, seq_len_min=300, num_q_heads=8,
                                         num_kv_heads=2)
    w = kvsynth.generate(rec)
    dev = upload(w)
    s = dev.shape
    full = host_f64(dev.bounds)
    dev.bounds.fill_(-7.0)
    sd.update_page_bounds(s, dev.k, dev.bt, dev.sl, dev.bounds,
                          pages=torch.zeros((0, 2), dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert np.all(host_f64(dev.bounds) == -7.0)
    U = [-(-int(n) // s.page_size) for n in w.seq_lens]
    listed = [(0, 0), (1, U[1] - 1), (2, 5), (0, U[0] - 1)]
    junk = [(0, U[0]), (1, s.max_pages_per_seq + 3), (3, 0), (-1, 2), (2, -4)]
    pages = torch.tensor(listed + junk, dtype=torch.int32).cuda()
    sd.update_page_bounds(s, dev.k, dev.bt, dev.sl, dev.bounds, pages=pages)
    torch.cuda.synchronize()
    got = host_f64(dev.bounds)
    mask = np.zeros(got.shape[:3], dtype=bool)
    for b, u in listed:
        mask[b, :, u] = True
    np.testing.assert_array_equal(got[mask], full[mask])
    assert np.all(got[~mask] == -7.0)
