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
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import kvsynth
import sparse_kv_cache_sd_amd as sd
from oracle import sdref

from gpu_util import GAP, TOL, oracle_group, upload

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
