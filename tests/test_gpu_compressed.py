"""GPU parity of the compressed-key page scorer (sd_update_compressed_keys,
sd_score_compressed, and sd_decode_step_sel with scorer "compressed").

Rules:
* window means: within the fp32 rounding of a sum of at most 32 keys,
  (32 + 2) * 2^-24 * max |K| of the window's head;
* page scores: against the oracle's formula applied to the library's own
  window means, within the fp32 rounding of the summed query and the
  d-term product, (d + 2G + 8) * 2^-24 * scale * sum_c (sum_h |q_hc|) |c_c|;
* whole steps: the kept set equals the oracle's (fp64 windows) where its
  score gap at k exceeds 1e-4, else is a valid top-k within 1e-4 and the
  outputs are compared with the oracle rerun on it; out / lse max-abs 2e-2
  (bf16) or 1e-5 (fp32).
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import kvsynth
import sparse_kv_cache_sd_amd as sd
from oracle import sdref

from gpu_util import GAP, TOL, check_selection, upload

pytestmark = pytest.mark.gpu

R = kvsynth.RECIPES
EPS = 2.0 ** -24


def _ckeys(dev):
    ck = torch.full(sd.compressed_keys_shape(dev.shape), float("nan"), dtype=torch.float32,
                    device="cuda")
    sd.update_compressed_keys(dev.shape, dev.k, dev.bt, dev.sl, ck)
    torch.cuda.synchronize()
    return ck


def _oracle_group(w, b, g, r_kv, scale, kept_override=None, selection=None):
    r = w.recipe
    G = r.group
    n = int(w.seq_lens[b])
    return sdref.group_step(sdref.widen(w.q[b, g * G:(g + 1) * G], r.dtype),
                            sdref.widen(w.K[b, g, :n], r.dtype), sdref.widen(w.V[b, g, :n], r.dtype),
                            unit="page", page_size=r.page_size, r_kv=r_kv, scale=scale,
                            kept_override=kept_override, selection=selection, scorer="compressed")


CASES = [
    ("l70b-20k", R["l70b"].with_(seq_len=20000)),
    ("l8b-6k", R["l8b"].with_(seq_len=6000, num_q_heads=16, num_kv_heads=4)),
    ("batch-ragged", R["batch"].with_(batch=4, seq_len=5000, seq_len_min=1, num_q_heads=16,
                                      num_kv_heads=4)),
    ("f32-d64", R["l8b"].with_(seq_len=3000, dtype="f32", head_dim=64, num_q_heads=8,
                               num_kv_heads=2)),
    ("g1-p64", R["l70b"].with_(seq_len=3000, num_q_heads=4, num_kv_heads=4)),
]


@pytest.mark.parametrize("cid,rec", CASES, ids=[c[0] for c in CASES])
def test_compressed_keys_and_scores(cid, rec):
    w = kvsynth.generate(rec)
    dev = upload(w)
    s = dev.shape
    scale = 1.0 / math.sqrt(s.head_dim)
    ck = _ckeys(dev).cpu().numpy().astype(np.float64)
    scores = torch.full((s.batch, s.num_kv_heads, s.max_pages_per_seq), float("nan"),
                        dtype=torch.float32, device="cuda")
    sd.score_compressed(s, dev.q, torch.from_numpy(ck.astype(np.float32)).cuda(), dev.sl, scores)
    torch.cuda.synchronize()
    sc = scores.cpu().numpy().astype(np.float64)
    G = s.group
    for b in range(s.batch):
        n = int(w.seq_lens[b])
        J = -(-n // 16)
        U = sdref.num_units(n, "page", s.page_size)
        for g in range(s.num_kv_heads):
            K = sdref.widen(w.K[b, g, :n], s.dtype)
            ref = sdref.compressed_keys(K)
            kmax = np.abs(K).max()
            np.testing.assert_allclose(ck[b, g, :J], ref, rtol=0, atol=34 * EPS * kmax)
            qg = sdref.widen(w.q[b, g * G:(g + 1) * G], s.dtype)
            want = sdref.compressed_page_scores(qg, ck[b, g, :J], s.page_size, scale)
            bound_w = (s.head_dim + 2 * G + 8) * EPS * scale * (np.abs(ck[b, g, :J]) @
                                                                np.abs(qg).sum(axis=0))
            per = s.page_size // 16
            bound = np.array([bound_w[u * per:(u + 1) * per].max() for u in range(U)])
            err = np.abs(sc[b, g, :U] - want)
            assert np.all(err <= bound + 1e-30), f"(b={b}, g={g}) score error {err.max()}"


@pytest.mark.parametrize("kind", ["topk", "init_local_topk"])
@pytest.mark.parametrize("cid,rec", CASES[:4], ids=[c[0] for c in CASES[:4]])
def test_decode_with_compressed_scorer(cid, rec, kind):
    w = kvsynth.generate(rec)
    dev = upload(w)
    s = dev.shape
    scale = 1.0 / math.sqrt(s.head_dim)
    r = 0.05 if s.page_size == 64 else 0.2
    sel = sd.Selection(kind, r, 1 if kind != "topk" else 0, 4 if kind != "topk" else 0,
                       scorer="compressed")
    osel = sdref.Selection(kind, r, sel.init_units, sel.local_units)
    ck = _ckeys(dev)
    cap = sd.selection_capacity(sel, s.max_pages_per_seq)
    ws = sd.alloc_workspace_sel(s, "page", sel)
    out = torch.empty((s.batch, s.num_q_heads, s.head_dim), dtype=torch.float32, device="cuda")
    lse = torch.empty((s.batch, s.num_q_heads), dtype=torch.float32, device="cuda")
    idx = torch.full((s.batch, s.num_kv_heads, cap), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((s.batch, s.num_kv_heads), -7, dtype=torch.int32, device="cuda")
    sd.decode_step_sel(s, dev.q, dev.k, dev.v, ck, dev.bt, dev.sl, "page", sel, out, lse, ws,
                       sel_idx=idx, sel_count=cnt)
    torch.cuda.synchronize()
    out, lse, idx, cnt = out.cpu().numpy(), lse.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy()
    G, tol = s.group, TOL[s.dtype]
    for b in range(s.batch):
        for g in range(s.num_kv_heads):
            orc = _oracle_group(w, b, g, r, scale, selection=osel)
            c = int(cnt[b, g])
            kept = idx[b, g, :c].astype(np.int64)
            if kind == "topk":
                exact = check_selection(kept, orc)
            else:
                exact = orc.gap > GAP
                if exact:
                    np.testing.assert_array_equal(kept, orc.kept)
            if not exact:
                orc = _oracle_group(w, b, g, r, scale, kept_override=kept)
            heads = slice(g * G, (g + 1) * G)
            e_o = float(np.abs(out[b, heads] - orc.out_sparse).max())
            e_l = float(np.abs(lse[b, heads] - orc.lse_sparse).max())
            assert e_o <= tol and e_l <= tol, f"(b={b}, g={g}) out {e_o} lse {e_l}"
