"""GPU parity of the structured index sets: the KV window, and the union of
initial, local and top-k units, through sd_select_units and
sd_decode_step_sel.

Rules (as in gpu_util):
* kept lists: bit-exact.  A window depends on no score.  The union is
  checked against the oracle's union rule applied to the library's own fp32
  unit scores (its top-k is exact on those), and also against the oracle's
  fp64 union wherever the oracle's score gap at k exceeds 1e-4;
* out / lse: max-abs <= 1e-5 (fp32 data) or 2e-2 (bf16 data) against the
  oracle's attention over the kept set.
Cases cover the fused page path (bf16, the attention blocks select the union
themselves), the listed page path (fp32), token unit with one-block and
many-block top-k, ragged batches, forced ranges wider than the sequence and
sequences of a single unit.

Dropped-mass budget (token unit): the kept list must be exactly the top-k of
the library's own scores at the chosen count; the count must equal the
oracle's wherever the oracle's dropped mass at that count and one fewer is
more than 1e-5 from the target (and the score gaps exceed 1e-4), and must
otherwise be valid with the oracle's fp64 masses: within the target (unless
capped) and one unit fewer not.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import kvsynth
import sparse_kv_cache_sd_amd as sd
from oracle import sdref

from gpu_util import GAP, TOL, oracle_group, random_shapes, upload

pytestmark = pytest.mark.gpu

R = kvsynth.RECIPES


def _gpu_scores(dev, unit):
    s = dev.shape
    scores = torch.empty((s.batch, s.num_kv_heads, s.units_max(unit)), dtype=torch.float32,
                         device="cuda")
    logits = (torch.empty((s.batch, s.num_q_heads, s.max_seq_len), dtype=torch.float32,
                          device="cuda") if unit == "token" else None)
    sd.score_pages(s, dev.q, dev.k, dev.bounds, dev.bt, dev.sl, unit, scores, logits)
    torch.cuda.synchronize()
    return scores.cpu().numpy().astype(np.float64)


def _expected_on_own_scores(sc, U, sel):
    if U == 0:
        return np.zeros(0, dtype=np.int64)
    return sdref.selected_units(sc[:U], sdref.Selection(sel.kind, sel.r_kv, sel.init_units,
                                                        sel.local_units))


def _run(dev, unit, sel):
    s = dev.shape
    cap = sd.selection_capacity(sel, s.units_max(unit))
    ws = sd.alloc_workspace_sel(s, unit, sel)
    out = torch.empty((s.batch, s.num_q_heads, s.head_dim), dtype=torch.float32, device="cuda")
    lse = torch.empty((s.batch, s.num_q_heads), dtype=torch.float32, device="cuda")
    idx = torch.full((s.batch, s.num_kv_heads, cap), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((s.batch, s.num_kv_heads), -7, dtype=torch.int32, device="cuda")
    sd.decode_step_sel(s, dev.q, dev.k, dev.v, dev.bounds, dev.bt, dev.sl, unit, sel, out, lse,
                       ws, sel_idx=idx, sel_count=cnt)
    idx2 = torch.full_like(idx, -7)
    cnt2 = torch.full_like(cnt, -7)
    scores = None
    if sel.kind != "window":
        scores = torch.empty((s.batch, s.num_kv_heads, s.units_max(unit)), dtype=torch.float32,
                             device="cuda")
        logits = (torch.empty((s.batch, s.num_q_heads, s.max_seq_len), dtype=torch.float32,
                              device="cuda") if unit == "token" else None)
        sd.score_pages(s, dev.q, dev.k, dev.bounds, dev.bt, dev.sl, unit, scores, logits)
    sd.select_units(s, unit, dev.sl, scores, sel, idx2, cnt2, ws=ws)
    torch.cuda.synchronize()
    return (out.cpu().numpy(), lse.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy(),
            idx2.cpu().numpy(), cnt2.cpu().numpy())


def _check(dev, unit, sel, groups=None):
    w, s = dev.w, dev.shape
    scale = 1.0 / math.sqrt(s.head_dim)
    out, lse, idx, cnt, idx2, cnt2 = _run(dev, unit, sel)
    own = None if sel.kind == "window" else _gpu_scores(dev, unit)
    G, tol = s.group, TOL[s.dtype]
    osel = sdref.Selection(sel.kind, sel.r_kv, sel.init_units, sel.local_units)
    if groups is None:
        groups = [(b, g) for b in range(s.batch) for g in range(s.num_kv_heads)]
    worst = 0.0
    for b, g in groups:
        n = int(w.seq_lens[b])
        U = sdref.num_units(n, unit, s.page_size)
        exp = (sdref.window_set(U, sel.r_kv) if own is None
               else _expected_on_own_scores(own[b, g], U, sel))
        c = int(cnt[b, g])
        assert c == exp.size, f"(b={b}, g={g}) count {c} != {exp.size}"
        kept = idx[b, g, :c].astype(np.int64)
        np.testing.assert_array_equal(kept, exp, err_msg=f"decode_step_sel (b={b}, g={g})")
        assert int(cnt2[b, g]) == c
        np.testing.assert_array_equal(idx2[b, g, :c], exp, err_msg=f"select_units (b={b}, g={g})")
        orc = oracle_group(w, b, g, unit, sel.r_kv, scale, kept_override=kept)
        if own is not None and orc.gap > GAP:
            np.testing.assert_array_equal(kept, sdref.selected_units(orc.sigma, osel))
        heads = slice(g * G, (g + 1) * G)
        e_o = float(np.abs(out[b, heads] - orc.out_sparse).max())
        e_l = float(np.abs(lse[b, heads] - orc.lse_sparse).max())
        assert e_o <= tol and e_l <= tol, f"(b={b}, g={g}) out {e_o} lse {e_l} > {tol}"
        worst = max(worst, e_o, e_l)
    return worst


SEL = sd.Selection

CASES = [
    # fused page path: the attention blocks select the union
    ("l8b-union", R["l8b"].with_(seq_len=6000, num_q_heads=16, num_kv_heads=4), "page",
     SEL("init_local_topk", 0.2, 1, 8)),
    ("l8b-union-none-forced", R["l8b"].with_(seq_len=6000, num_q_heads=16, num_kv_heads=4),
     "page", SEL("init_local_topk", 0.2, 0, 0)),
    ("l8b-union-all-forced", R["l8b"].with_(seq_len=900, num_q_heads=8, num_kv_heads=2), "page",
     SEL("init_local_topk", 0.05, 40, 30)),
    ("l70b-union", R["l70b"].with_(seq_len=20000), "page", SEL("init_local_topk", 0.05, 1, 32)),
    ("batch-union", R["batch"].with_(batch=4, seq_len=5000, seq_len_min=1, num_kv_heads=4,
                                     num_q_heads=16), "page", SEL("init_local_topk", 0.2, 2, 5)),
    ("l8b-window", R["l8b"].with_(seq_len=6000, num_q_heads=16, num_kv_heads=4), "page",
     SEL("window", 0.3)),
    ("batch-window", R["batch"].with_(batch=4, seq_len=5000, seq_len_min=1, num_kv_heads=4,
                                      num_q_heads=16), "page", SEL("window", 0.2)),
    ("l8b-topk", R["l8b"].with_(seq_len=6000, num_q_heads=16, num_kv_heads=4), "page",
     SEL("topk", 0.3)),
    # listed page path (fp32 data)
    ("f32-page-union", R["l8b"].with_(seq_len=3000, dtype="f32", num_q_heads=8, num_kv_heads=2,
                                      head_dim=64), "page", SEL("init_local_topk", 0.1, 3, 4)),
    ("f32-page-window", R["l8b"].with_(seq_len=3000, dtype="f32", num_q_heads=8, num_kv_heads=2,
                                       head_dim=64), "page", SEL("window", 0.1)),
    # token unit: one-block and many-block top-k
    ("tiny-union", R["tiny"], "token", SEL("init_local_topk", 0.25, 4, 64)),
    ("tiny-window", R["tiny"], "token", SEL("window", 0.25)),
    ("sweep-union", R["sweep"].with_(seq_len=3000, num_q_heads=8, num_kv_heads=2), "token",
     SEL("init_local_topk", 0.2, 16, 128)),
    ("sweep-union-many-block", R["sweep"].with_(seq_len=20000, num_q_heads=8, num_kv_heads=2),
     "token", SEL("init_local_topk", 0.1, 4, 1024)),
    ("sweep-window", R["sweep"].with_(seq_len=20000, num_q_heads=8, num_kv_heads=2), "token",
     SEL("window", 0.2)),
]


@pytest.mark.parametrize("cid,rec,unit,sel", CASES, ids=[c[0] for c in CASES])
def test_structured_matches_oracle(cid, rec, unit, sel):
    print(f"[structured] {cid}", flush=True)
    dev = upload(kvsynth.generate(rec))
    worst = _check(dev, unit, sel)
    print(f"[structured] {cid}: max-abs {worst:.2e}", flush=True)


def _random_structured(n, seed):
    """Seeded random shapes (gpu_util.random_shapes, no empty sequences) with
    a window, a union of random forced ranges, or the plain top-k."""
    rng = np.random.default_rng(seed + 1)
    out = []
    for cid, kw, unit, r, _ in random_shapes(n, seed, allow_empty=False, max_len=20000):
        kind = str(rng.choice(["window", "init_local_topk", "topk"]))
        r = min(r, 0.9)
        if kind == "init_local_topk":
            sel = SEL(kind, r, int(rng.integers(0, 5)), int(rng.integers(0, 65)))
        else:
            sel = SEL(kind, r)
        out.append((f"{cid}-{kind}", kw, unit, sel))
    return out


RANDOM_CASES = _random_structured(12, 3030)


@pytest.mark.parametrize("cid,kw,unit,sel", RANDOM_CASES, ids=[c[0] for c in RANDOM_CASES])
def test_structured_random_shapes(cid, kw, unit, sel):
    print(f"[structured] {cid}", flush=True)
    dev = upload(kvsynth.generate(R["batch"].with_(**kw)))
    _check(dev, unit, sel)


@pytest.mark.parametrize("unit,P", [("page", 16), ("page", 64), ("token", 16)])
def test_single_unit_sequences(unit, P):
    rec = R["l8b"].with_(batch=3, seq_len=P if unit == "page" else 1, seq_len_min=1,
                         page_size=P, num_q_heads=8, num_kv_heads=2)
    dev = upload(kvsynth.generate(rec))
    for sel in (SEL("init_local_topk", 0.3, 1, 1), SEL("window", 0.3)):
        _check(dev, unit, sel)


def test_selection_rejects():
    rec = R["l8b"].with_(seq_len=500, num_q_heads=8, num_kv_heads=2)
    dev = upload(kvsynth.generate(rec))
    s = dev.shape
    for bad in (SEL("init_local_topk", 0.3, -1, 0), SEL("window", 0.0), SEL("sliding", 0.3)):
        with pytest.raises((sd.SdError, ValueError)):
            sd.workspace_bytes_sel(s, "page", bad)


# ---------------------------------------------------------------- dropped-mass budget

MARGIN = 1e-5   # fp32 softmax weights summed in 2^-40 fixed point vs the fp64 oracle


def _budget_run(dev, sel):
    s = dev.shape
    cap = sd.selection_capacity(sel, s.max_seq_len)
    ws = sd.alloc_workspace_sel(s, "token", sel)
    out = torch.empty((s.batch, s.num_q_heads, s.head_dim), dtype=torch.float32, device="cuda")
    lse = torch.empty((s.batch, s.num_q_heads), dtype=torch.float32, device="cuda")
    idx = torch.full((s.batch, s.num_kv_heads, cap), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((s.batch, s.num_kv_heads), -7, dtype=torch.int32, device="cuda")
    sd.decode_step_sel(s, dev.q, dev.k, dev.v, None, dev.bt, dev.sl, "token", sel, out, lse, ws,
                       sel_idx=idx, sel_count=cnt)
    scores = torch.empty((s.batch, s.num_kv_heads, s.max_seq_len), dtype=torch.float32,
                         device="cuda")
    logits = torch.empty((s.batch, s.num_q_heads, s.max_seq_len), dtype=torch.float32,
                         device="cuda")
    sd.score_pages(s, dev.q, dev.k, dev.bounds, dev.bt, dev.sl, "token", scores, logits)
    idx2 = torch.full_like(idx, -7)
    cnt2 = torch.full_like(cnt, -7)
    sd.select_units(s, "token", dev.sl, scores, sel, idx2, cnt2, ws=ws, token_logits=logits)
    torch.cuda.synchronize()
    return (out.cpu().numpy(), lse.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy(),
            idx2.cpu().numpy(), cnt2.cpu().numpy(), scores.cpu().numpy().astype(np.float64))


def _check_budget(dev, sel, groups=None):
    """Every (b, g), or the listed ones: the count against the oracle's rule,
    the list against the top-k of the library's own scores at that count, the
    output against the oracle on the kept set."""
    w, s = dev.w, dev.shape
    scale = 1.0 / math.sqrt(s.head_dim)
    out, lse, idx, cnt, idx2, cnt2, own = _budget_run(dev, sel)
    G, tol = s.group, TOL[s.dtype]
    exact = 0
    for b in range(s.batch):
        n = int(w.seq_lens[b])
        cap = sdref.keep_count(sel.r_kv, n)
        for g in range(s.num_kv_heads):
            if groups is not None and (b, g) not in groups:
                continue
            k = int(cnt[b, g])
            assert 1 <= k <= cap, f"(b={b}, g={g}) count {k} outside [1, {cap}]"
            kept = idx[b, g, :k].astype(np.int64)
            # the list is the exact top-k of the library's own scores at that count
            np.testing.assert_array_equal(kept, sdref.select_topk(own[b, g, :n], k)[0])
            assert int(cnt2[b, g]) == k
            np.testing.assert_array_equal(idx2[b, g, :k], kept)
            # the count against the oracle's fp64 masses
            qg = sdref.widen(w.q[b, g * G:(g + 1) * G], s.dtype)
            Kg = sdref.widen(w.K[b, g, :n], s.dtype)
            sg = sdref.group_logits(qg, Kg, scale)
            worst = lambda T: max(sdref.dropped_mass(sg[h], T) for h in range(G))
            if k < cap:
                assert worst(kept) <= sel.max_dropped + MARGIN
            if k > 1:
                fewer = sdref.select_topk(own[b, g, :n], k - 1)[0]
                assert worst(fewer) > sel.max_dropped - MARGIN
            k_or = sdref.mass_budget_count(sg, sg.max(axis=0), sel.max_dropped, cap)
            sig = sg.max(axis=0)
            clear = True
            for kk in (k_or - 1, k_or):
                if 1 <= kk < n:
                    top, gap = sdref.select_topk(sig, kk)
                    clear &= gap > 1e-4 and abs(worst(top) - sel.max_dropped) > MARGIN
            if clear:
                assert k == k_or, f"(b={b}, g={g}) count {k} != oracle {k_or}"
                exact += 1
            orc = oracle_group(w, b, g, "token", sel.r_kv, scale, kept_override=kept)
            heads = slice(g * G, (g + 1) * G)
            e_o = float(np.abs(out[b, heads] - orc.out_sparse).max())
            e_l = float(np.abs(lse[b, heads] - orc.lse_sparse).max())
            assert e_o <= tol and e_l <= tol, f"(b={b}, g={g}) out {e_o} lse {e_l} > {tol}"
    return exact


BUDGET_CASES = [
    ("tiny", R["tiny"], [0.01, 0.1, 0.3]),
    ("sweep-3k", R["sweep"].with_(seq_len=3000, num_q_heads=8, num_kv_heads=2), [0.02, 0.2]),
    ("sweep-20k", R["sweep"].with_(seq_len=20000, num_q_heads=8, num_kv_heads=2), [0.05]),
    ("g8-ragged", R["l70b"].with_(batch=3, seq_len=4000, seq_len_min=1, num_q_heads=16,
                                  num_kv_heads=2), [0.1]),
    ("sweep-32k", R["sweep"].with_(seq_len=32768, num_q_heads=8, num_kv_heads=2), [0.1]),
    # the switch between one and many blocks per (b, g)
    ("sweep-8192", R["sweep"].with_(seq_len=8192, num_q_heads=8, num_kv_heads=2), [0.1]),
    ("sweep-8193", R["sweep"].with_(seq_len=8193, num_q_heads=8, num_kv_heads=2), [0.1]),
    # past 8192 tokens the budget runs over many blocks per (b, g): 40
    # slices with a ragged last one, and a ragged G = 8 batch
    ("sweep-40k", R["sweep"].with_(seq_len=40000, num_q_heads=8, num_kv_heads=2), [0.05, 0.3]),
    ("g8-ragged-70k", R["l70b"].with_(batch=3, seq_len=70000, seq_len_min=1, num_q_heads=16,
                                      num_kv_heads=2), [0.1]),
]


@pytest.mark.parametrize("cid,rec,targets", BUDGET_CASES, ids=[c[0] for c in BUDGET_CASES])
def test_mass_budget_matches_oracle(cid, rec, targets):
    print(f"[budget] {cid}", flush=True)
    dev = upload(kvsynth.generate(rec))
    for t in targets:
        exact = _check_budget(dev, sd.Selection("mass_budget", 0.5, max_dropped=t))
        print(f"[budget] {cid} target {t}: {exact} counts equal to the oracle's", flush=True)


def test_mass_budget_edges():
    rec = R["sweep"].with_(seq_len=2000, num_q_heads=8, num_kv_heads=2)
    dev = upload(kvsynth.generate(rec))
    s = dev.shape
    # target 1: one unit; target 0: the cap
    for t, want in ((1.0, 1), (0.0, sdref.keep_count(0.3, 2000))):
        out, lse, idx, cnt, *_ = _budget_run(dev, sd.Selection("mass_budget", 0.3, max_dropped=t))
        assert np.all(cnt == want)
    # without a cap (r_kv >= 1) the budget still decides the count
    out, lse, idx, cnt, *_ = _budget_run(dev, sd.Selection("mass_budget", 1.0, max_dropped=0.2))
    assert np.all((cnt >= 1) & (cnt < 2000))
    # page unit and too many tokens are refused
    with pytest.raises(sd.SdError):
        sd.workspace_bytes_sel(s, "page", sd.Selection("mass_budget", 0.3, max_dropped=0.1))
        ws = sd.alloc_workspace_sel(s, "page", sd.Selection("mass_budget", 0.3, max_dropped=0.1))
        out = torch.empty((s.batch, s.num_q_heads, s.head_dim), dtype=torch.float32, device="cuda")
        lse = torch.empty((s.batch, s.num_q_heads), dtype=torch.float32, device="cuda")
        sd.decode_step_sel(s, dev.q, dev.k, dev.v, dev.bounds, dev.bt, dev.sl, "page",
                           sd.Selection("mass_budget", 0.3, max_dropped=0.1), out, lse, ws)
    with pytest.raises(sd.SdError):
        sd.workspace_bytes_sel(s, "token", sd.Selection("mass_budget", 0.3, max_dropped=1.5))


def test_mass_budget_edges_many_blocks():
    """Targets 1 and 0 past 32768 tokens (the many-block kernels), with an
    empty and a one-token sequence in the batch."""
    rec = R["sweep"].with_(batch=3, seq_len=40000, num_q_heads=8, num_kv_heads=2)
    w = kvsynth.generate(rec, seq_lens=[40000, 0, 1])
    dev = upload(w)
    for t in (1.0, 0.0):
        out, lse, idx, cnt, *_ = _budget_run(dev, sd.Selection("mass_budget", 0.3, max_dropped=t))
        for b, n in enumerate(w.seq_lens):
            want = 0 if n == 0 else (1 if t == 1.0 else sdref.keep_count(0.3, int(n)))
            assert np.all(cnt[b] == want), (t, b, cnt[b], want)
        assert np.all(idx[2, :, 0] == 0)


@pytest.mark.parametrize("max_seq,tied", [(1001, False), (1001, True), (4096, True),
                                           (40000, False), (40000, True)])
def test_mass_budget_on_given_logits(max_seq, tied):
    """sd_select_units on hand-made logits (rows of any length, heavy ties in
    the group score): the count against the oracle's rule on the same fp32
    values, and the list the top-k at that count."""
    rng = np.random.default_rng(max_seq + tied)
    B, Hq, Hkv, G = 2, 8, 2, 4
    lens = np.array([max_seq, max_seq // 2 + 3], dtype=np.int32)
    lg = (rng.standard_normal((B, Hq, max_seq)) * 1.5).astype(np.float32)
    if tied:
        lg = np.round(lg * 2.0) / 2.0
    sig = lg.reshape(B, Hkv, G, max_seq).max(axis=2).astype(np.float32)
    P = 16
    s = sd.Shape(B, Hq, Hkv, 64, P, -(-max_seq // P), max_seq, "f32", 64)
    for t in (0.02, 0.2):
        sel = sd.Selection("mass_budget", 0.6, max_dropped=t)
        cap_row = sd.selection_capacity(sel, max_seq)
        idx = torch.full((B, Hkv, cap_row), -7, dtype=torch.int32, device="cuda")
        cnt = torch.full((B, Hkv), -7, dtype=torch.int32, device="cuda")
        ws = sd.alloc_workspace_sel(s, "token", sel)
        sd.select_units(s, "token", torch.from_numpy(lens).cuda(), torch.from_numpy(sig).cuda(),
                        sel, idx, cnt, ws=ws, token_logits=torch.from_numpy(lg).cuda())
        torch.cuda.synchronize()
        idx, cnt = idx.cpu().numpy(), cnt.cpu().numpy()
        for b in range(B):
            n = int(lens[b])
            cap = sdref.keep_count(0.6, n)
            for g in range(Hkv):
                sg = lg[b, g * G:(g + 1) * G, :n].astype(np.float64)
                sgm = sig[b, g, :n].astype(np.float64)
                k = int(cnt[b, g])
                np.testing.assert_array_equal(idx[b, g, :k], sdref.select_topk(sgm, k)[0])
                worst = lambda kk: max(sdref.dropped_mass(sg[h], sdref.select_topk(sgm, kk)[0])
                                       for h in range(G))
                assert 1 <= k <= cap
                if k < cap:
                    assert worst(k) <= t + MARGIN
                if k > 1:
                    assert worst(k - 1) > t - MARGIN
                k_or = sdref.mass_budget_count(sg, sgm, t, cap)
                if all(abs(worst(kk) - t) > MARGIN for kk in (k_or - 1, k_or) if 1 <= kk < n):
                    assert k == k_or
