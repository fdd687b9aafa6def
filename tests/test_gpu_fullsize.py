"""Full-size GPU parity: every decode configuration at its real size, through
one ``sd.decode_step`` call in the launch configuration the benchmark times
(default split plan and workspace).

Two kinds of check:

* sampled (sequence, KV head) instances against the fp64 oracle, under the
  rules of ``gpu_util`` (selected sets bit-exact where the oracle's score gap
  at k exceeds 1e-4, out / lse max-abs 2e-2 for bf16);
* for every instance, properties that hold at any size: the count follows the
  keep-count rule, and the kept ids are exactly the top-k of the library's own
  fp32 unit scores (equal scores to the lower id, ascending), which is unique;
  every output is finite.
"""

from __future__ import annotations

import functools
import math

import numpy as np
import pytest
import torch

import kvsynth
import sparse_kv_cache_sd_amd as sd
from oracle import sdref

from gpu_util import compare_step, own_topk_property, run_decode, upload

pytestmark = pytest.mark.gpu

K = kvsynth.KTOK


@functools.lru_cache(maxsize=2)
def _dev(name: str, context: int | None):
    if name == "l8b":
        rec = kvsynth.RECIPES["l8b"]
    elif name == "sweep":
        rec = kvsynth.sweep_recipe(context, 0.3)
    elif name == "batch":
        rec = kvsynth.RECIPES["batch"]
    elif name == "l70b":
        rec = kvsynth.l70b_recipe(context)
    else:
        raise ValueError(name)
    print(f"[fullsize] generating {name} context={context}", flush=True)
    return upload(kvsynth.generate(rec))


def _finite(out, lse):
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))


# (id, recipe name, context, unit, r_kv, sampled (b, g) instances or "all",
#  instances whose oracle score gap at k exceeds 1e-4, so that their kept set
#  is compared exactly; the rest take the gap rule's fallback.  Counted from
#  the oracle on these seeded inputs: a drop means the comparison got weaker)
CASES = [
    ("l8b-32k-page-0.3", "l8b", None, "page", 0.3, "all", 8),
    ("l8b-32k-dense", "l8b", None, "page", 1.0, [(0, 0), (0, 5)], 0),
    ("sweep-128k-token-0.3", "sweep", 128 * K, "token", 0.3, [(0, 0), (0, 3), (0, 7)], 1),
    ("sweep-128k-token-0.2", "sweep", 128 * K, "token", 0.2, [(0, 1), (0, 6)], 0),
    ("sweep-128k-dense", "sweep", 128 * K, "token", 1.0, [(0, 2)], 0),
    ("sweep-64k-token-0.2", "sweep", 64 * K, "token", 0.2, [(0, 4)], 0),
    ("sweep-32k-token-0.3", "sweep", 32 * K, "token", 0.3, "all", 2),
    ("sweep-32k-token-0.2", "sweep", 32 * K, "token", 0.2, "all", 2),
    ("sweep-8k-token-0.3", "sweep", 8 * K, "token", 0.3, "all", 8),
    ("sweep-2k-token-0.2", "sweep", 2 * K, "token", 0.2, "all", 8),
    ("l70b-128k-page-0.05", "l70b", 128 * K, "page", 0.05, "all", 8),
    ("batch-page-0.2", "batch", None, "page", 0.2, "extremes", 4),
    ("l70b-1m-page-0.05", "l70b", 1024 * K, "page", 0.05, [(0, 0), (0, 7)], 1),
]


@pytest.mark.parametrize("cid,name,context,unit,r_kv,groups,n_exact", CASES,
                         ids=[c[0] for c in CASES])
def test_full_size(cid, name, context, unit, r_kv, groups, n_exact):
    print(f"[fullsize] {cid}", flush=True)
    dev = _dev(name, context)
    s = dev.shape
    if groups == "all":
        groups = [(b, g) for b in range(s.batch) for g in range(s.num_kv_heads)]
    elif groups == "extremes":
        lens = dev.w.seq_lens
        groups = [(int(np.argmin(lens)), 0), (int(np.argmax(lens)), 7), (3, 2), (11, 5)]
    if r_kv < 1.0:
        out, lse, sel, cnt = run_decode(dev, unit, r_kv)
        _finite(out, lse)
        own_topk_property(dev, unit, r_kv, sel, cnt)
    counts = {}
    e_o, e_l = compare_step(dev, unit, r_kv, groups=groups, counts=counts)
    assert counts.get("exact", 0) == n_exact, counts
    print(f"[fullsize] {cid}: {len(groups)} instances vs oracle ({counts.get('exact', 0)} as "
          f"exact sets, {counts.get('fallback', 0)} under the gap rule), max-abs out {e_o:.2e} "
          f"lse {e_l:.2e}", flush=True)


# ---------------------------------------------------------------- alpha-entmax

def _entmax_step(dev, unit: str, r_kv: float, alpha: float):
    s = dev.shape
    sel = sd.Selection("topk", r_kv)
    cap = sd.selection_capacity(sel, s.units_max(unit))
    ws = sd.alloc_workspace_entmax(s, unit, sel)
    out = torch.full((s.batch, s.num_q_heads, s.head_dim), float("nan"), device="cuda")
    tau = torch.full((s.batch, s.num_q_heads), float("nan"), device="cuda")
    idx = torch.full((s.batch, s.num_kv_heads, cap), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((s.batch, s.num_kv_heads), -7, dtype=torch.int32, device="cuda")
    sd.decode_step_entmax(s, dev.q, dev.k, dev.v, dev.bounds, dev.bt, dev.sl, unit, sel, alpha,
                          out, ws, tau=tau, sel_idx=idx, sel_count=cnt)
    torch.cuda.synchronize()
    return out.cpu().numpy(), tau.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy()


ENTMAX_CASES = [
    ("l8b-32k-page-0.3", "l8b", None, "page", 0.3, "all"),
    ("sweep-128k-token-0.3", "sweep", 128 * K, "token", 0.3, [(0, 2), (0, 5)]),
    ("l70b-128k-page-0.05", "l70b", 128 * K, "page", 0.05, "all"),
    ("batch-page-0.2", "batch", None, "page", 0.2, "extremes"),
    ("l70b-1m-page-0.05", "l70b", 1024 * K, "page", 0.05, [(0, 3)]),
]


@pytest.mark.parametrize("cid,name,context,unit,r_kv,groups", ENTMAX_CASES,
                         ids=[c[0] for c in ENTMAX_CASES])
def test_full_size_entmax(cid, name, context, unit, r_kv, groups):
    """1.5-entmax over the kept set at full size: the kept lists are the
    softmax path's (the top-k of the library's own scores for every
    instance), and sampled instances match the fp64 entmax oracle (gap rule
    for the set; out max-abs 2e-2, tau 1e-3)."""
    from oracle import entmaxref
    from gpu_util import GAP, check_selection
    print(f"[fullsize] entmax {cid}", flush=True)
    alpha = 1.5
    dev = _dev(name, context)
    s, w = dev.shape, dev.w
    out, tau, idx, cnt = _entmax_step(dev, unit, r_kv, alpha)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(tau))
    own_topk_property(dev, unit, r_kv, idx, cnt)
    if groups == "all":
        groups = [(b, g) for b in range(s.batch) for g in range(s.num_kv_heads)]
    elif groups == "extremes":
        lens = w.seq_lens
        groups = [(int(np.argmin(lens)), 0), (int(np.argmax(lens)), 7)]
    G, scale = s.group, 1.0 / math.sqrt(s.head_dim)
    e_o = e_t = 0.0
    for b, g in groups:
        n = int(w.seq_lens[b])
        args = (sdref.widen(w.q[b, g * G:(g + 1) * G], s.dtype), sdref.widen(w.K[b, g, :n], s.dtype),
                sdref.widen(w.V[b, g, :n], s.dtype))
        kw = dict(unit=unit, page_size=s.page_size, r_kv=r_kv, scale=scale, alpha=alpha)
        orc = entmaxref.group_step(*args, **kw)
        kept = idx[b, g, :int(cnt[b, g])].astype(np.int64)
        if not check_selection(kept, orc):
            orc = entmaxref.group_step(*args, kept_override=kept, **kw)
        heads = slice(g * G, (g + 1) * G)
        eo = float(np.abs(out[b, heads] - orc.out_sparse).max())
        et = float(np.abs(tau[b, heads] - orc.tau_sparse).max())
        assert eo <= 2e-2 and et <= 1e-3, f"(b={b}, g={g}) out {eo} tau {et}"
        e_o, e_t = max(e_o, eo), max(e_t, et)
    print(f"[fullsize] entmax {cid}: {len(groups)} instances vs oracle, max-abs out {e_o:.2e} "
          f"tau {e_t:.2e}", flush=True)


# ------------------------------------------- structured sets, budget, compressed scorer

def _structured_cases():
    SEL = sd.Selection
    return [
        # the bench's union at 32K: 1 initial + 2048 tokens of local pages + top-k r 0.3
        ("l8b-32k-union", "l8b", None, "page", SEL("init_local_topk", 0.3, 1, 128), "all"),
        ("l8b-32k-window", "l8b", None, "page", SEL("window", 0.3), "all"),
        # SparDA App. C's setup at 1M: 1 initial block, a 2048-token window, 96 blocks
        ("l70b-1m-appc", "l70b", 1024 * K, "page",
         SEL("init_local_topk", 96 / 16384, 1, 32), [(0, 1), (0, 6)]),
    ]


@pytest.mark.parametrize("cid,name,context,unit,sel,groups", _structured_cases(),
                         ids=[c[0] for c in _structured_cases()])
def test_full_size_structured(cid, name, context, unit, sel, groups):
    """Kept lists bit-exact against the oracle's rule on the library's own
    scores (and on the oracle's fp64 scores where the gap rule applies), for
    every instance or the sampled ones; outputs against the oracle."""
    from test_gpu_structured import _check
    print(f"[fullsize] {cid}", flush=True)
    dev = _dev(name, context)
    worst = _check(dev, unit, sel, groups=None if groups == "all" else groups)
    print(f"[fullsize] {cid}: max-abs {worst:.2e}", flush=True)


@pytest.mark.parametrize("target,cap", [(0.05, 0.5), (0.6, 0.9)], ids=["bench", "binding"])
def test_full_size_mass_budget(target, cap):
    """The dropped-mass budget at 32K token, every instance: the bench's
    setting (at most 5% of each head's softmax mass dropped, capped at r 0.5,
    where these inputs reach the cap) and one where the target binds below
    the cap."""
    from test_gpu_structured import _check_budget
    print(f"[fullsize] sweep-32k budget {target} cap {cap}", flush=True)
    dev = _dev("sweep", 32 * K)
    exact = _check_budget(dev, sd.Selection("mass_budget", cap, max_dropped=target))
    print(f"[fullsize] sweep-32k budget {target} cap {cap}: {exact} counts equal to the "
          f"oracle's", flush=True)


def test_full_size_mass_budget_128k():
    """The dropped-mass budget at 128K token (many blocks per (b, g)), the
    target binding below the cap; sampled instances against the oracle."""
    from test_gpu_structured import _check_budget
    print("[fullsize] sweep-128k budget 0.3 cap 0.9", flush=True)
    dev = _dev("sweep", 128 * K)
    exact = _check_budget(dev, sd.Selection("mass_budget", 0.9, max_dropped=0.3),
                          groups=[(0, 0), (0, 3), (0, 7)])
    print(f"[fullsize] sweep-128k budget: {exact} counts equal to the oracle's", flush=True)


@pytest.mark.parametrize("cid,name,context,r_kv,groups", [
    ("l8b-32k-compressed", "l8b", None, 0.3, "all"),
    ("l70b-128k-compressed", "l70b", 128 * K, 0.05, [(0, 0), (0, 4), (0, 7)]),
], ids=["l8b-32k-compressed", "l70b-128k-compressed"])
def test_full_size_compressed_scorer(cid, name, context, r_kv, groups):
    """The compressed-key scorer's step at full size: kept pages under the gap
    rule against the oracle's compressed scorer (fp64 windows), outputs
    against the oracle on the kept set."""
    from gpu_util import TOL, check_selection
    print(f"[fullsize] {cid}", flush=True)
    dev = _dev(name, context)
    s, w = dev.shape, dev.w
    ck = torch.empty(sd.compressed_keys_shape(s), dtype=torch.float32, device="cuda")
    sd.update_compressed_keys(s, dev.k, dev.bt, dev.sl, ck)
    sel = sd.Selection("topk", r_kv, scorer="compressed")
    cap = sd.selection_capacity(sel, s.max_pages_per_seq)
    ws = sd.alloc_workspace_sel(s, "page", sel)
    out = torch.empty((s.batch, s.num_q_heads, s.head_dim), device="cuda")
    lse = torch.empty((s.batch, s.num_q_heads), device="cuda")
    idx = torch.full((s.batch, s.num_kv_heads, cap), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((s.batch, s.num_kv_heads), -7, dtype=torch.int32, device="cuda")
    sd.decode_step_sel(s, dev.q, dev.k, dev.v, ck, dev.bt, dev.sl, "page", sel, out, lse, ws,
                       sel_idx=idx, sel_count=cnt)
    torch.cuda.synchronize()
    out, lse, idx, cnt = out.cpu().numpy(), lse.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy()
    _finite(out, lse)
    if groups == "all":
        groups = [(b, g) for b in range(s.batch) for g in range(s.num_kv_heads)]
    G, scale, tol = s.group, 1.0 / math.sqrt(s.head_dim), TOL[s.dtype]
    worst = 0.0
    for b, g in groups:
        n = int(w.seq_lens[b])
        args = (sdref.widen(w.q[b, g * G:(g + 1) * G], s.dtype), sdref.widen(w.K[b, g, :n], s.dtype),
                sdref.widen(w.V[b, g, :n], s.dtype))
        kw = dict(unit="page", page_size=s.page_size, r_kv=r_kv, scale=scale, scorer="compressed")
        orc = sdref.group_step(*args, **kw)
        kept = idx[b, g, :int(cnt[b, g])].astype(np.int64)
        if not check_selection(kept, orc):
            orc = sdref.group_step(*args, kept_override=kept, **kw)
        heads = slice(g * G, (g + 1) * G)
        e_o = float(np.abs(out[b, heads] - orc.out_sparse).max())
        e_l = float(np.abs(lse[b, heads] - orc.lse_sparse).max())
        assert e_o <= tol and e_l <= tol, f"(b={b}, g={g}) out {e_o} lse {e_l}"
        worst = max(worst, e_o, e_l)
    print(f"[fullsize] {cid}: {len(groups)} instances, max-abs {worst:.2e}", flush=True)
