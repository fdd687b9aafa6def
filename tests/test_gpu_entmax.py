"""GPU parity of alpha-entmax attention over the kept set (sd_decode_step_entmax)
against the fp64 oracle (oracle/entmaxref.py).

Rules:
* kept lists: as for the softmax step (the same scorers and top-k): equal to
  the oracle's where its score gap at k exceeds 1e-4, else a valid top-k
  within 1e-4, and the outputs are compared with the oracle rerun on the
  GPU's own set;
* out: max-abs <= 1e-5 (fp32 data) or 2e-2 (bf16 data);
* tau: the thresholds solve the same equation over logits that the GPU
  accumulates in fp32, so they are compared within 1e-5 (fp32) or 1e-3
  (bf16, where the logits of bf16 data carry fp32 summation error of up to
  about d * 2^-24 * scale * sum |q K|);
* a sequence with no attended token gives out = 0 and tau = +inf.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import kvsynth
import sparse_kv_cache_sd_amd as sd
from oracle import entmaxref, sdref

from gpu_util import GAP, TOL, check_selection, random_shapes, upload

pytestmark = pytest.mark.gpu

R = kvsynth.RECIPES
TAU_TOL = {"f32": 1e-5, "bf16": 1e-3}


def _run(dev, unit, sel, alpha, stats=None):
    s = dev.shape
    umax = s.units_max(unit)
    cap = sd.selection_capacity(sel, umax)
    ws = sd.alloc_workspace_entmax(s, unit, sel)
    ws.fill_(0xA5)  # contents need not be initialised
    out = torch.full((s.batch, s.num_q_heads, s.head_dim), float("nan"), device="cuda")
    tau = torch.full((s.batch, s.num_q_heads), float("nan"), device="cuda")
    idx = torch.full((s.batch, s.num_kv_heads, cap), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((s.batch, s.num_kv_heads), -7, dtype=torch.int32, device="cuda")
    sd.decode_step_entmax(s, dev.q, dev.k, dev.v, dev.bounds if stats is None else stats, dev.bt,
                          dev.sl, unit, sel, alpha, out, ws, tau=tau, sel_idx=idx, sel_count=cnt)
    torch.cuda.synchronize()
    return out.cpu().numpy(), tau.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy()


def _oracle(w, b, g, unit, r_kv, scale, alpha, kept_override=None, selection=None):
    r = w.recipe
    G = r.group
    n = int(w.seq_lens[b])
    return entmaxref.group_step(sdref.widen(w.q[b, g * G:(g + 1) * G], r.dtype),
                                sdref.widen(w.K[b, g, :n], r.dtype),
                                sdref.widen(w.V[b, g, :n], r.dtype),
                                unit=unit, page_size=r.page_size, r_kv=r_kv, scale=scale,
                                alpha=alpha, kept_override=kept_override, selection=selection)


def _compare(w, dev, unit, sel, alpha, res, groups=None):
    """Checks every (b, g) of ``groups`` (default all); returns max errors."""
    out, tau, idx, cnt = res
    s = dev.shape
    G, tol = s.group, TOL[s.dtype]
    scale = 1.0 / math.sqrt(s.head_dim)
    dense = sel.r_kv >= 1.0 and sel.kind != "mass_budget"
    osel = sdref.Selection(sel.kind, sel.r_kv, sel.init_units, sel.local_units, sel.max_dropped)
    if groups is None:
        groups = [(b, g) for b in range(s.batch) for g in range(s.num_kv_heads)]
    e_out = e_tau = 0.0
    for b, g in groups:
        heads = slice(g * G, (g + 1) * G)
        if int(w.seq_lens[b]) == 0:
            assert np.all(out[b, heads] == 0.0) and np.all(np.isposinf(tau[b, heads]))
            continue
        orc = _oracle(w, b, g, unit, sel.r_kv, scale, alpha, selection=osel)
        if dense:
            ref_o, ref_t = orc.out_dense, orc.tau_dense
        else:
            c = int(cnt[b, g])
            kept = idx[b, g, :c].astype(np.int64)
            if sel.kind == "topk":
                exact = check_selection(kept, orc)
            elif sel.kind == "window":
                np.testing.assert_array_equal(kept, orc.kept)
                exact = True
            else:
                exact = orc.gap > GAP
                if exact:
                    np.testing.assert_array_equal(kept, orc.kept)
            if not exact:
                orc = _oracle(w, b, g, unit, sel.r_kv, scale, alpha, kept_override=kept)
            ref_o, ref_t = orc.out_sparse, orc.tau_sparse
        eo = float(np.abs(out[b, heads] - ref_o).max())
        et = float(np.abs(tau[b, heads] - ref_t).max())
        assert eo <= tol, f"(b={b}, g={g}) out max-abs {eo} > {tol}"
        assert et <= TAU_TOL[s.dtype], f"(b={b}, g={g}) tau max-abs {et}"
        e_out, e_tau = max(e_out, eo), max(e_tau, et)
    return e_out, e_tau


CASES = [
    # name, recipe, unit, r_kv
    ("tiny-token", R["tiny"], "token", 0.25),
    ("l8b-6k-page", R["l8b"].with_(seq_len=6000, num_q_heads=16, num_kv_heads=4), "page", 0.3),
    ("l8b-5k-token", R["l8b"].with_(seq_len=5000, num_q_heads=16, num_kv_heads=4), "token", 0.2),
    ("l70b-20k-page", R["l70b"].with_(seq_len=20000), "page", 0.05),
    ("f32-d64-page", R["l8b"].with_(seq_len=3000, dtype="f32", head_dim=64, num_q_heads=8,
                                    num_kv_heads=2), "page", 0.3),
    ("g1-p64-token", R["l70b"].with_(seq_len=3001, num_q_heads=4, num_kv_heads=4), "token", 0.1),
    ("batch-ragged-page", R["batch"].with_(batch=4, seq_len=5000, seq_len_min=1, num_q_heads=16,
                                           num_kv_heads=4), "page", 0.2),
]


@pytest.mark.parametrize("alpha", [1.5, 2.0, 1.25])
@pytest.mark.parametrize("cid,rec,unit,r", CASES, ids=[c[0] for c in CASES])
def test_entmax_topk(cid, rec, unit, r, alpha):
    w = kvsynth.generate(rec)
    dev = upload(w)
    sel = sd.Selection("topk", r)
    _compare(w, dev, unit, sel, alpha, _run(dev, unit, sel, alpha))


@pytest.mark.parametrize("unit", ["token", "page"])
@pytest.mark.parametrize("cid,rec", [("l8b-4k", R["l8b"].with_(seq_len=4000, num_q_heads=16,
                                                                num_kv_heads=4)),
                                      ("f32-d64", R["l8b"].with_(seq_len=2000, dtype="f32",
                                                                 head_dim=64, num_q_heads=8,
                                                                 num_kv_heads=2))],
                         ids=["l8b-4k", "f32-d64"])
def test_entmax_dense(cid, rec, unit):
    w = kvsynth.generate(rec)
    dev = upload(w)
    sel = sd.Selection("topk", 1.0)
    _compare(w, dev, unit, sel, 1.5, _run(dev, unit, sel, 1.5))


@pytest.mark.parametrize("kind", ["window", "init_local_topk"])
@pytest.mark.parametrize("unit", ["token", "page"])
def test_entmax_structured(kind, unit):
    rec = R["l8b"].with_(seq_len=4500, num_q_heads=16, num_kv_heads=4)
    w = kvsynth.generate(rec)
    dev = upload(w)
    local = 64 if unit == "token" else 4
    sel = sd.Selection(kind, 0.2, 1 if kind != "window" else 0, local if kind != "window" else 0)
    _compare(w, dev, unit, sel, 1.5, _run(dev, unit, sel, 1.5))


@pytest.mark.parametrize("n", [3000, 20000])
def test_entmax_mass_budget(n):
    # 20000 tokens: the budget over many blocks per (b, g)
    rec = R["l8b"].with_(seq_len=n, num_q_heads=8, num_kv_heads=2)
    w = kvsynth.generate(rec)
    dev = upload(w)
    sel = sd.Selection("mass_budget", 0.5, max_dropped=0.2)
    out, tau, idx, cnt = _run(dev, "token", sel, 1.5)
    s = dev.shape
    G = s.group
    scale = 1.0 / math.sqrt(s.head_dim)
    # the budget's count is checked by the softmax tests; here the entmax
    # outputs over the GPU's own kept list
    for g in range(s.num_kv_heads):
        assert 1 <= int(cnt[0, g]) <= sdref.keep_count(0.5, n)
        kept = idx[0, g, :int(cnt[0, g])].astype(np.int64)
        assert np.all(np.diff(kept) > 0) and kept[0] >= 0 and kept[-1] < n
        orc = _oracle(w, 0, g, "token", 0.5, scale, 1.5, kept_override=kept)
        heads = slice(g * G, (g + 1) * G)
        assert np.abs(out[0, heads] - orc.out_sparse).max() <= TOL["bf16"]
        assert np.abs(tau[0, heads] - orc.tau_sparse).max() <= TAU_TOL["bf16"]


def test_entmax_support_recovery_is_exact():
    """The tiny needle inputs: the token top-k at r = 0.25 holds every head's
    1.5-entmax support (pinned in the oracle tests), so the sparse GPU output
    matches the oracle's DENSE entmax output."""
    rec = R["tiny"]
    w = kvsynth.generate(rec)
    dev = upload(w)
    out, tau, idx, cnt = _run(dev, "token", sd.Selection("topk", rec.r_kv), 1.5)
    n = int(w.seq_lens[0])
    orc = _oracle(w, 0, 0, "token", rec.r_kv, 1.0 / math.sqrt(rec.head_dim), 1.5)
    assert np.all(orc.delta == 0.0)
    assert np.abs(out[0] - orc.out_dense).max() <= TOL["f32"]
    assert np.abs(tau[0] - orc.tau_dense).max() <= TAU_TOL["f32"]
    assert n == 1024


def test_entmax_long_kept_list():
    """More than 32768 kept tokens per head: the threshold kernel re-reads the
    logits beyond its registers."""
    rec = R["tiny"].with_(seq_len=40000, seed=21)
    w = kvsynth.generate(rec)
    dev = upload(w)
    sel = sd.Selection("topk", 0.9)
    res = _run(dev, "token", sel, 1.5)
    assert int(res[3][0, 0]) == 36000
    _compare(w, dev, "token", sel, 1.5, res)


def test_entmax_empty_and_short_sequences():
    rec = R["l8b"].with_(batch=5, seq_len=70, num_q_heads=8, num_kv_heads=2)
    w = kvsynth.generate(rec, seq_lens=np.array([5, 1, 17, 64, 70], dtype=np.int32))
    dev = upload(w)
    dev.sl[0] = 0      # an empty sequence (the oracle side reads w.seq_lens)
    w.seq_lens[0] = 0
    for unit in ("token", "page"):
        sel = sd.Selection("topk", 0.5)
        _compare(w, dev, unit, sel, 1.5, _run(dev, unit, sel, 1.5))
        sel = sd.Selection("topk", 1.0)
        _compare(w, dev, unit, sel, 1.5, _run(dev, unit, sel, 1.5))


def test_entmax_deterministic_and_workspace_reuse():
    rec = R["l8b"].with_(seq_len=6000, num_q_heads=16, num_kv_heads=4)
    w = kvsynth.generate(rec)
    dev = upload(w)
    sel = sd.Selection("topk", 0.3)
    a = _run(dev, "page", sel, 1.5)
    b = _run(dev, "page", sel, 1.5)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_entmax_rejects_bad_alpha():
    rec = R["l8b"].with_(seq_len=100, num_q_heads=8, num_kv_heads=2)
    dev = upload(kvsynth.generate(rec))
    sel = sd.Selection("topk", 0.5)
    for bad in (1.0, 0.9, 2.5, float("nan")):
        with pytest.raises(sd.SdError, match="SD_E_RATIO"):
            _run(dev, "page", sel, bad)


@pytest.mark.parametrize("alpha", [1.5, 1.25])
def test_entmax_flat_logits_many_candidates(alpha):
    """q = 0: every logit is 0, every kept token is a candidate and the weights
    are uniform.  With 36000 kept tokens the threshold kernel holds 16384 in
    registers and has more candidates per thread than its LDS slots, so it
    re-reads the rest each step."""
    rec = R["tiny"].with_(seq_len=40000, seed=22)
    w = kvsynth.generate(rec)
    w.q[...] = 0
    dev = upload(w)
    sel = sd.Selection("topk", 0.9)
    res = _run(dev, "token", sel, alpha)
    _compare(w, dev, "token", sel, alpha, res)
    k = int(res[3][0, 0])
    # tau solves k * (-tau)^beta = 1
    want = -(1.0 / k) ** (alpha - 1.0)
    assert np.abs(res[1][0] - want).max() <= 1e-6


@pytest.mark.parametrize("cid,rec", [
    ("l70b-20k", R["l70b"].with_(seq_len=20000)),
    ("l8b-6k", R["l8b"].with_(seq_len=6000, num_q_heads=16, num_kv_heads=4)),
], ids=["l70b-20k", "l8b-6k"])
def test_entmax_with_compressed_scorer(cid, rec):
    """Entmax over the pages the compressed-key scorer keeps (the fused page
    path selects them from those scores)."""
    w = kvsynth.generate(rec)
    dev = upload(w)
    s = dev.shape
    ck = torch.empty(sd.compressed_keys_shape(s), dtype=torch.float32, device="cuda")
    sd.update_compressed_keys(s, dev.k, dev.bt, dev.sl, ck)
    r = 0.05 if s.page_size == 64 else 0.3
    sel = sd.Selection("topk", r, scorer="compressed")
    out, tau, idx, cnt = _run(dev, "page", sel, 1.5, stats=ck)
    G, scale = s.group, 1.0 / math.sqrt(s.head_dim)
    for g in range(s.num_kv_heads):
        n = int(w.seq_lens[0])
        args = (sdref.widen(w.q[0, g * G:(g + 1) * G], s.dtype), sdref.widen(w.K[0, g, :n], s.dtype),
                sdref.widen(w.V[0, g, :n], s.dtype))
        # the kept pages against the oracle's compressed scorer (gap rule)
        soft = sdref.group_step(*args, unit="page", page_size=s.page_size, r_kv=r, scale=scale,
                                scorer="compressed")
        kept = idx[0, g, :int(cnt[0, g])].astype(np.int64)
        check_selection(kept, soft)
        orc = entmaxref.group_step(*args, unit="page", page_size=s.page_size, r_kv=r,
                                   scale=scale, alpha=1.5, kept_override=kept)
        heads = slice(g * G, (g + 1) * G)
        assert np.abs(out[0, heads] - orc.out_sparse).max() <= TOL[s.dtype]
        assert np.abs(tau[0, heads] - orc.tau_sparse).max() <= TAU_TOL[s.dtype]


def test_entmax_token_ragged_batch():
    rec = R["batch"].with_(batch=4, seq_len=5000, seq_len_min=1, num_q_heads=16, num_kv_heads=4,
                           unit="token")
    w = kvsynth.generate(rec)
    dev = upload(w)
    for r in (0.2, 1.0):
        sel = sd.Selection("topk", r)
        _compare(w, dev, "token", sel, 1.5, _run(dev, "token", sel, 1.5))


@pytest.mark.parametrize("alpha", [1.5, 1.25])
@pytest.mark.parametrize("seq_len", [6000, 65536], ids=["lds-newton", "block-fallback"])
def test_entmax_flat_logits_bf16_pages(seq_len, alpha):
    """q = 0 on bf16 pages: every logit is 0 and every kept token is a
    candidate.  At 6000 tokens (1808 kept slots per head) the candidates are
    too many for the Newton steps in registers and run in LDS; at 65536
    tokens (19664 slots) the threshold is split into chunks whose candidate
    lists overflow, so the whole block iterates over every kept logit."""
    rec = R["l8b"].with_(seq_len=seq_len, num_q_heads=16, num_kv_heads=4)
    w = kvsynth.generate(rec)
    w.q[...] = 0
    dev = upload(w)
    sel = sd.Selection("topk", 0.3)
    res = _run(dev, "page", sel, alpha)
    _compare(w, dev, "page", sel, alpha, res)
    _, tau, idx, cnt = res
    P, G = rec.page_size, rec.group
    for g in range(rec.num_kv_heads):
        pages = idx[0, g, :int(cnt[0, g])].astype(np.int64)
        n = int(np.minimum(P, seq_len - pages * P).sum())
        # tau solves n * (-tau)^beta = 1
        want = -(1.0 / n) ** (alpha - 1.0)
        assert np.abs(tau[0, g * G:(g + 1) * G] - want).max() <= 1e-6


def _random_entmax(n, seed):
    """Seeded random shapes (gpu_util.random_shapes) with a random alpha and a
    top-k, window or union selection."""
    rng = np.random.default_rng(seed + 1)
    out = []
    for cid, kw, unit, r, empty in random_shapes(n, seed, max_len=20000):
        kind = str(rng.choice(["topk", "window", "init_local_topk"]))
        alpha = float(rng.choice([1.25, 1.5, 2.0]))
        if kind == "init_local_topk":
            sel = sd.Selection(kind, min(r, 0.9), int(rng.integers(0, 5)),
                               int(rng.integers(0, 65)))
        else:
            sel = sd.Selection(kind, r)
        out.append((f"{cid}-{kind}-a{alpha}", kw, unit, sel, alpha, empty))
    return out


RANDOM_CASES = _random_entmax(12, 4040)


@pytest.mark.parametrize("cid,kw,unit,sel,alpha,empty", RANDOM_CASES,
                         ids=[c[0] for c in RANDOM_CASES])
def test_entmax_random_shapes(cid, kw, unit, sel, alpha, empty):
    print(f"[entmax] {cid}", flush=True)
    w = kvsynth.generate(R["batch"].with_(**kw))
    dev = upload(w)
    if empty:  # the oracle and the library both see length 0
        w.seq_lens[-1] = 0
        dev.sl[-1] = 0
    _compare(w, dev, unit, sel, alpha, _run(dev, unit, sel, alpha))
