"""Helpers for the GPU parity tests: upload a kvsynth workload and compare the
HIP path with the oracle under the stated rules.

Comparison rules
* integer and index outputs: bit-exact;
* a selection instance (sequence b, KV head g) whose oracle score gap at the
  k-th unit exceeds 1e-4 must select exactly the oracle's set; otherwise
  every kept unit must score >= sigma_(k) - 1e-4 and every dropped unit
  <= sigma_(k) + 1e-4, and the outputs are compared with the oracle rerun
  on the GPU's own set;
* outputs and lse: max-abs <= 1e-5 for fp32 data, <= 2e-2 for bf16 data;
* scores: within the fp32 rounding bound (d + 4) * 2^-24 * scale * sum_c |q_c x_c|
  of a d-term dot product accumulated in fp32.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
import torch

import kvsynth
import sparse_kv_cache_sd_amd as sd
from oracle import sdref

GAP = 1e-4
TOL = {"f32": 1e-5, "bf16": 2e-2}


def t_dev(a: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def host_f64(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        bits = t.cpu().view(torch.int16).numpy().view(np.uint16)
        return sdref.widen(bits, "bf16")
    return t.cpu().double().numpy()


@dataclass
class Dev:
    w: kvsynth.Workload
    shape: sd.Shape
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    bt: torch.Tensor
    sl: torch.Tensor
    bounds: torch.Tensor


def upload(w: kvsynth.Workload, softmax_scale: float = 0.0) -> Dev:
    r = w.recipe
    pc = w.paged()
    shape = sd.Shape(r.batch, r.num_q_heads, r.num_kv_heads, r.head_dim, r.page_size,
                     w.max_pages(), w.n_alloc, r.dtype, pc.num_pages, softmax_scale)
    dt = torch.float32 if r.dtype == "f32" else torch.bfloat16
    bounds = torch.zeros(sd.bounds_shape(shape), dtype=dt, device="cuda")
    dev = Dev(w, shape, t_dev(w.q, r.dtype), t_dev(pc.k_pool, r.dtype), t_dev(pc.v_pool, r.dtype),
              torch.from_numpy(pc.block_table).cuda(), torch.from_numpy(w.seq_lens).cuda(), bounds)
    sd.update_page_bounds(shape, dev.k, dev.bt, dev.sl, dev.bounds)
    return dev


def run_decode(dev: Dev, unit: str, r_kv: float):
    s = dev.shape
    ws = sd.alloc_workspace(s, unit, r_kv)
    out = torch.empty((s.batch, s.num_q_heads, s.head_dim), dtype=torch.float32, device="cuda")
    lse = torch.empty((s.batch, s.num_q_heads), dtype=torch.float32, device="cuda")
    sel = cnt = None
    if r_kv < 1.0:
        k_max = sd.keep_count(r_kv, s.units_max(unit))
        sel = torch.full((s.batch, s.num_kv_heads, k_max), -7, dtype=torch.int32, device="cuda")
        cnt = torch.full((s.batch, s.num_kv_heads), -7, dtype=torch.int32, device="cuda")
    sd.decode_step(s, dev.q, dev.k, dev.v, dev.bounds, dev.bt, dev.sl, unit, r_kv, out, lse, ws,
                   sel_idx=sel, sel_count=cnt)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy(), (None if sel is None else sel.cpu().numpy()), \
        (None if cnt is None else cnt.cpu().numpy())


def oracle_group(w: kvsynth.Workload, b: int, g: int, unit: str, r_kv: float, scale: float,
                 kept_override=None):
    r = w.recipe
    G = r.group
    n = int(w.seq_lens[b])
    qg = sdref.widen(w.q[b, g * G:(g + 1) * G], r.dtype)
    Kg = sdref.widen(w.K[b, g, :n], r.dtype)
    Vg = sdref.widen(w.V[b, g, :n], r.dtype)
    return sdref.group_step(qg, Kg, Vg, unit=unit, page_size=r.page_size, r_kv=r_kv,
                            scale=scale, kept_override=kept_override)


def check_selection(gpu_kept: np.ndarray, orc: sdref.GroupResult) -> bool:
    """Returns True when the sets must be (and are) identical; False when the
    gap rule allowed a different valid set (asserted valid here)."""
    if orc.gap > GAP:
        np.testing.assert_array_equal(gpu_kept, orc.kept)
        return True
    k = orc.k
    assert gpu_kept.size == k and np.all(np.diff(gpu_kept) > 0)
    kth = np.sort(orc.sigma)[::-1][k - 1]
    dropped = np.setdiff1d(np.arange(orc.sigma.size), gpu_kept)
    assert np.all(orc.sigma[gpu_kept] >= kth - GAP)
    assert np.all(orc.sigma[dropped] <= kth + GAP)
    return False


def compare_step(dev: Dev, unit: str, r_kv: float, groups=None, report=None, counts=None):
    """Run the whole decode step on the GPU and compare every (b, g) in
    ``groups`` (default all) with the oracle.  Returns the max errors.
    ``counts`` (a dict), if given, receives how many instances were compared
    as exact sets ("exact", oracle gap > 1e-4) and how many under the gap
    rule's fallback ("fallback")."""
    w, s = dev.w, dev.shape
    scale = 1.0 / math.sqrt(s.head_dim) if s.softmax_scale <= 0 else s.softmax_scale
    out, lse, sel, cnt = run_decode(dev, unit, r_kv)
    G, tol = s.group, TOL[s.dtype]
    if groups is None:
        groups = [(b, g) for b in range(s.batch) for g in range(s.num_kv_heads)]
    err_o = err_l = 0.0
    for b, g in groups:
        heads = slice(g * G, (g + 1) * G)
        if int(w.seq_lens[b]) == 0:
            # an empty sequence keeps nothing and gives out = 0, lse = -inf
            # (the oracle takes no empty instance)
            assert np.all(out[b, heads] == 0) and np.all(np.isneginf(lse[b, heads]))
            if r_kv < 1.0:
                assert int(cnt[b, g]) == 0
            continue
        orc = oracle_group(w, b, g, unit, r_kv, scale)
        if r_kv >= 1.0:
            ref_o, ref_l = orc.out_dense, orc.lse_dense
        else:
            assert int(cnt[b, g]) == orc.k
            kept = sel[b, g, :orc.k].astype(np.int64)
            exact = check_selection(kept, orc)
            if counts is not None:
                key = "exact" if exact else "fallback"
                counts[key] = counts.get(key, 0) + 1
            if exact:
                ref_o, ref_l = orc.out_sparse, orc.lse_sparse
            else:
                o2 = oracle_group(w, b, g, unit, r_kv, scale, kept_override=kept)
                ref_o, ref_l = o2.out_sparse, o2.lse_sparse
        e_o = float(np.abs(out[b, heads] - ref_o).max())
        e_l = float(np.abs(lse[b, heads] - ref_l).max())
        assert e_o <= tol, f"(b={b}, g={g}) out max-abs {e_o} > {tol}"
        assert e_l <= tol, f"(b={b}, g={g}) lse max-abs {e_l} > {tol}"
        err_o, err_l = max(err_o, e_o), max(err_l, e_l)
    if report is not None:
        report.append((unit, r_kv, err_o, err_l))
    return err_o, err_l


def own_topk_property(dev, unit: str, r_kv: float, sel: np.ndarray, cnt: np.ndarray):
    """The kept set of every (b, g) is the top-k of the library's own unit
    scores, ties to the lower id, in ascending order."""
    s = dev.shape
    umax = s.units_max(unit)
    scores = torch.empty((s.batch, s.num_kv_heads, umax), dtype=torch.float32, device="cuda")
    logits = (torch.empty((s.batch, s.num_q_heads, s.max_seq_len), dtype=torch.float32,
                          device="cuda") if unit == "token" else None)
    sd.score_pages(s, dev.q, dev.k, dev.bounds, dev.bt, dev.sl, unit, scores, logits)
    torch.cuda.synchronize()
    sc = scores.cpu().numpy()
    P = s.page_size
    for b in range(s.batch):
        n = int(dev.w.seq_lens[b])
        U = -(-n // P) if unit == "page" else n
        k = sdref.keep_count(r_kv, U)
        assert int(cnt[b].min()) == k and int(cnt[b].max()) == k, f"b={b}: count != {k}"
        for g in range(s.num_kv_heads):
            x = sc[b, g, :U].astype(np.float64)
            assert np.all(np.isfinite(x))
            ref = np.sort(np.lexsort((np.arange(U), -x))[:k])
            np.testing.assert_array_equal(sel[b, g, :k], ref, err_msg=f"(b={b}, g={g})")


def random_shapes(n, seed, allow_empty=True, max_len=36000):
    """n seeded random decode-step shapes the library accepts: (id, recipe
    keyword arguments for the "batch" recipe, unit, r_kv, empty) with batch
    1-4, G and H_kv in {1, 2, 4, 8}, d in {64, 128}, pages of 16 or 64 tokens,
    bf16 or fp32, ragged lengths up to max_len, and (empty) the last sequence
    of a batch to be emptied by the caller."""
    rng = np.random.default_rng(seed)
    lens = [x for x in (300, 2000, 9000, 20000, 36000) if x <= max_len]
    out = []
    for i in range(n):
        G = int(rng.choice([1, 2, 4, 8]))
        Hkv = int(rng.choice([1, 2, 4, 8]))
        d = int(rng.choice([64, 128]))
        P = int(rng.choice([16, 64]))
        dtype = "f32" if rng.random() < 0.25 else "bf16"
        B = int(rng.integers(1, 5))
        unit = "token" if rng.random() < 0.5 else "page"
        n_max = int(rng.choice(lens))
        n_min = int(rng.integers(1, n_max + 1)) if B > 1 else n_max
        r = float(rng.choice([0.02, 0.1, 0.3, 0.5, 0.9, 1.0]))
        empty = allow_empty and B > 1 and rng.random() < 0.3
        out.append((f"{i:02d}-B{B}-G{G}-H{Hkv}-d{d}-P{P}-{dtype}-{unit}-n{n_max}-r{r}"
                    + ("-empty" if empty else ""),
                    dict(batch=B, num_q_heads=G * Hkv, num_kv_heads=Hkv, head_dim=d,
                         page_size=P, dtype=dtype, seq_len=n_max, seq_len_min=n_min,
                         seed=seed + i), unit, r, empty))
    return out
