"""GPU dropped mass delta (sd_dropped_mass, token unit) against the fp64
oracle (oracle.sdref.dropped_mass) on the GPU's own kept lists.

delta is the dense softmax mass of the attended tokens left out of a kept
list ([Cross/cards] pre-hoc sparsity abstract).  The GPU sums fp32 weights
of its own fp32 logits; those differ from the fp64 logits by at most the
derived accumulation bound (d + 4) 2^-24 scale sum |q K| (a few 1e-6 here),
which moves each weight by that relative amount, so delta is compared within
2e-4 relative plus 1e-6 absolute.  Also checked: a kept list holding every
token gives 0, an empty sequence gives 0, and the budget's lists leave at
most their target outside (unless capped).
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import kvsynth
import sparse_kv_cache_sd_amd as sd
from oracle import sdref

from gpu_util import upload

pytestmark = pytest.mark.gpu

R = kvsynth.RECIPES


def _scores(dev):
    s = dev.shape
    scores = torch.empty((s.batch, s.num_kv_heads, s.max_seq_len), device="cuda")
    logits = torch.empty((s.batch, s.num_q_heads, s.max_seq_len), device="cuda")
    sd.score_pages(s, dev.q, dev.k, dev.bounds, dev.bt, dev.sl, "token", scores, logits)
    return scores, logits


def _delta(dev, logits, idx, cnt):
    s = dev.shape
    delta = torch.full((s.batch, s.num_q_heads), float("nan"), device="cuda")
    sd.dropped_mass(s, dev.sl, dev.bt, logits, idx, cnt, delta)
    torch.cuda.synchronize()
    return delta.cpu().numpy()


def _compare(dev, delta, idx, cnt):
    w, s = dev.w, dev.shape
    G, scale = s.group, 1.0 / math.sqrt(s.head_dim)
    worst = 0.0
    for b in range(s.batch):
        n = int(w.seq_lens[b])
        for g in range(s.num_kv_heads):
            heads = slice(g * G, (g + 1) * G)
            if n == 0:
                assert np.all(delta[b, heads] == 0.0)
                continue
            kept = idx[b, g, :int(cnt[b, g])].astype(np.int64)
            sg = sdref.group_logits(sdref.widen(w.q[b, g * G:(g + 1) * G], s.dtype),
                                    sdref.widen(w.K[b, g, :n], s.dtype), scale)
            for i in range(G):
                ref = sdref.dropped_mass(sg[i], kept)
                err = abs(float(delta[b, g * G + i]) - ref)
                assert err <= 1e-6 + 2e-4 * ref, f"(b={b}, h={g * G + i}) delta {delta[b, g * G + i]} vs {ref}"
                worst = max(worst, err)
    return worst


CASES = [
    ("tiny", R["tiny"], 0.25),
    ("sweep-5k", R["sweep"].with_(seq_len=5000, num_q_heads=16, num_kv_heads=4), 0.2),
    # rows of a length not a multiple of 4: the one-token-per-load path
    ("sweep-5001", R["sweep"].with_(seq_len=5001, num_q_heads=16, num_kv_heads=4), 0.2),
    ("g8-ragged", R["l70b"].with_(batch=3, seq_len=4000, seq_len_min=1, num_q_heads=16,
                                  num_kv_heads=2), 0.1),
    ("sweep-128k", kvsynth.sweep_recipe(128 * kvsynth.KTOK, 0.3), 0.3),
]


@pytest.mark.parametrize("cid,rec,r", CASES, ids=[c[0] for c in CASES])
def test_dropped_mass_matches_oracle(cid, rec, r):
    print(f"[dropped] {cid}", flush=True)
    dev = upload(kvsynth.generate(rec))
    s = dev.shape
    scores, logits = _scores(dev)
    k_max = sd.keep_count(r, s.max_seq_len)
    idx = torch.empty((s.batch, s.num_kv_heads, k_max), dtype=torch.int32, device="cuda")
    cnt = torch.empty((s.batch, s.num_kv_heads), dtype=torch.int32, device="cuda")
    ws = sd.alloc_workspace(s, "token", r)
    sd.select_topk(s, "token", dev.sl, scores, r, idx, cnt, ws)
    delta = _delta(dev, logits, idx, cnt)
    worst = _compare(dev, delta, idx.cpu().numpy(), cnt.cpu().numpy())
    print(f"[dropped] {cid}: max-abs {worst:.2e}, delta in [{delta.min():.3g}, {delta.max():.3g}]",
          flush=True)


def test_dropped_mass_edges():
    rec = R["sweep"].with_(batch=3, seq_len=3000, num_q_heads=8, num_kv_heads=2)
    w = kvsynth.generate(rec, seq_lens=np.array([3000, 17, 900], dtype=np.int32))
    dev = upload(w)
    dev.sl[1] = 0      # an empty sequence
    w.seq_lens[1] = 0
    s = dev.shape
    _, logits = _scores(dev)
    # every token kept: nothing dropped
    full = torch.arange(s.max_seq_len, dtype=torch.int32, device="cuda").expand(
        s.batch, s.num_kv_heads, s.max_seq_len).contiguous()
    cnt = dev.sl.view(-1, 1).expand(s.batch, s.num_kv_heads).contiguous().to(torch.int32)
    delta = _delta(dev, logits, full, cnt)
    assert np.all(delta == 0.0)
    # nothing kept: everything dropped
    none = torch.full((s.batch, s.num_kv_heads, 1), -1, dtype=torch.int32, device="cuda")
    zero = torch.zeros((s.batch, s.num_kv_heads), dtype=torch.int32, device="cuda")
    delta = _delta(dev, logits, none, zero)
    assert np.allclose(delta[[0, 2]], 1.0, atol=1e-6) and np.all(delta[1] == 0.0)
    # an arbitrary unordered list with out-of-range ids (ignored)
    rng = np.random.default_rng(3)
    lst = np.stack([np.stack([rng.permutation(3000)[:700] for _ in range(s.num_kv_heads)])
                    for _ in range(s.batch)]).astype(np.int32)
    lst[:, :, 0] = 5000
    idx = torch.from_numpy(lst).cuda()
    cnt = torch.full((s.batch, s.num_kv_heads), 700, dtype=torch.int32, device="cuda")
    delta = _delta(dev, logits, idx, cnt)
    kept = [[np.array([t for t in lst[b, g] if t < int(w.seq_lens[b])], dtype=np.int64)
             for g in range(s.num_kv_heads)] for b in range(s.batch)]
    G, scale = s.group, 1.0 / math.sqrt(s.head_dim)
    for b in (0, 2):
        n = int(w.seq_lens[b])
        for g in range(s.num_kv_heads):
            sg = sdref.group_logits(sdref.widen(w.q[b, g * G:(g + 1) * G], s.dtype),
                                    sdref.widen(w.K[b, g, :n], s.dtype), scale)
            for i in range(G):
                ref = sdref.dropped_mass(sg[i], kept[b][g])
                assert abs(float(delta[b, g * G + i]) - ref) <= 1e-6 + 2e-4 * ref


@pytest.mark.parametrize("n", [6000, 50000])
def test_dropped_mass_of_the_budget(n):
    """The budget keeps the shortest prefix leaving at most the target of every
    head's mass outside: delta on its lists is within the target (up to the
    fp32 decision margin) wherever the cap does not bind, and one unit fewer
    leaves more than the target for some head.  50000 tokens: the budget
    over many blocks per (b, g)."""
    rec = R["sweep"].with_(seq_len=n, num_q_heads=16, num_kv_heads=4)
    dev = upload(kvsynth.generate(rec))
    s = dev.shape
    scores, logits = _scores(dev)
    for target in (0.02, 0.2):
        sel = sd.Selection("mass_budget", 0.9, max_dropped=target)
        cap = sd.selection_capacity(sel, s.max_seq_len)
        idx = torch.empty((s.batch, s.num_kv_heads, cap), dtype=torch.int32, device="cuda")
        cnt = torch.empty((s.batch, s.num_kv_heads), dtype=torch.int32, device="cuda")
        ws = sd.alloc_workspace_sel(s, "token", sel)
        sd.select_units(s, "token", dev.sl, scores, sel, idx, cnt, ws=ws, token_logits=logits)
        delta = _delta(dev, logits, idx, cnt)
        c = cnt.cpu().numpy()
        for g in range(s.num_kv_heads):
            if c[0, g] < cap:
                assert delta[0, g * s.group:(g + 1) * s.group].max() <= target + 1e-5
        _compare(dev, delta, idx.cpu().numpy(), c)
        # one unit fewer (the top-k of the same scores at count - 1) leaves
        # more than the target for some head of the group
        own = scores.cpu().numpy().astype(np.float64)
        fewer = np.zeros(idx.shape, dtype=np.int32)
        fcnt = np.maximum(c - 1, 1).astype(np.int32)
        for g in range(s.num_kv_heads):
            fewer[0, g, :fcnt[0, g]] = sdref.select_topk(own[0, g, :n], int(fcnt[0, g]))[0]
        d_f = _delta(dev, logits, torch.from_numpy(fewer).cuda(), torch.from_numpy(fcnt).cuda())
        for g in range(s.num_kv_heads):
            if c[0, g] >= 2:
                assert d_f[0, g * s.group:(g + 1) * s.group].max() > target - 1e-5


def test_dropped_mass_rejects():
    rec = R["tiny"]
    dev = upload(kvsynth.generate(rec))
    s = dev.shape
    logits = torch.empty((s.batch, s.num_q_heads, s.max_seq_len), device="cuda")
    idx = torch.zeros((s.batch, s.num_kv_heads, 4), dtype=torch.int32, device="cuda")
    cnt = torch.zeros((s.batch, s.num_kv_heads), dtype=torch.int32, device="cuda")
    delta = torch.empty((s.batch, s.num_q_heads), device="cuda")
    with pytest.raises(ValueError):
        sd.dropped_mass(s, dev.sl, dev.bt, logits, idx[0], cnt, delta)
