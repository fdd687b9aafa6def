#!/usr/bin/env python3
"""Decode-attention benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload l8b]
                    [--selection topk|window|init_local_topk|mass_budget]
                    [--scorer bounds|compressed] [--attention softmax|entmax]
                    [--no-points] [--blocks N]

A step is one decode step of one attention layer: page-bound (or exact)
scoring, top-k selection under r_KV and split-K attention over the kept
units, merged by log-sum-exp.  Inputs are resident in HBM before timing
starts.

Timing protocol, per workload:
* L distinct layer caches, L chosen from the bytes the SPARSE step reads so
  that between two reads of one layer the steps read at least 4x the 256 MB
  Infinity Cache of other layers' data (layers past the first are device
  copies of it at their own addresses);
* W untimed warmup steps and one untimed pass over the L layers, then
  exactly K step-layers (step i on layer i mod L) captured in one HIP graph
  and replayed once, timed with HIP events on the launch stream;
* the same for the dense step (every unit kept, same kernels) and for the
  attention kernel alone.

Prints ONE JSON line: the metric (microseconds per decode-step-layer of the
main workload, lower is better), effective HBM GB/s on the algorithmic
bytes, the roofline of the dominant kernel (the split-K attention kernel),
the dense step, `points` (the other workloads of the 32K-1M range, each with
its step time, GB/s, dense time, speedup, byte bound and attention-kernel
fraction), and the fp64 CPU oracle timed on a bounded sample on the host
cores (sparse and dense steps apart, one thread too, with the dropped mass
delta).  Token-unit results also report the dropped softmax mass of layer
0's selection, computed on the GPU.  --blocks N runs N fresh processes and
reports paired dense/sparse ratios with an interval from resampling them.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
MALL_BYTES = 256 * 2 ** 20      # Infinity Cache
METRIC = "µs per decode-step-layer + effective HBM GB/s (% roofline) at 32K–1M, r_KV"

WORKLOADS = {
    # name: (recipe name, overrides, unit, r_kv, description)
    "l8b": ("l8b", {}, "page", 0.3,
            "Llama-3.1-8B-shaped layer, batch 1, 32 q / 8 kv heads, d 128, bf16 paged KV "
            "(page 16), 32K context, page-bound top-k r_KV=0.3, split-K over kept pages"),
    "sweep128k-0.3": ("sweep", {"seq_len": 131072, "seed": 7}, "token", 0.3,
                      "8B-shaped, batch 1, 128K, exact q.K token top-k r_KV=0.3"),
    "sweep128k-0.2": ("sweep", {"seq_len": 131072, "seed": 7}, "token", 0.2,
                      "8B-shaped, batch 1, 128K, exact q.K token top-k r_KV=0.2"),
    "sweep32k-0.2": ("sweep", {"seq_len": 32768, "seed": 5}, "token", 0.2,
                     "8B-shaped, batch 1, 32K, exact q.K token top-k r_KV=0.2"),
    "sweep32k-0.3": ("sweep", {"seq_len": 32768, "seed": 5}, "token", 0.3,
                     "8B-shaped, batch 1, 32K, exact q.K token top-k r_KV=0.3"),
    "batch": ("batch", {}, "page", 0.2,
              "16 sequences x U(48K,64K) context, 8B-shaped, page-bound top-k r_KV=0.2"),
    "l70b-128k": ("l70b", {"seq_len": 131072, "seed": 5}, "page", 0.05,
                  "Llama-3.1-70B-shaped layer on one GPU, 64 q / 8 kv heads, page 64, 128K, "
                  "page-bound top-k r_KV=0.05"),
    "l70b-1m": ("l70b", {"seq_len": 1048576, "seed": 6}, "page", 0.05,
                "Llama-3.1-70B-shaped layer on one GPU, page 64, 1M context, r_KV=0.05"),
}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------
# algorithmic byte model (what the method must move per decode-step-layer)
# ----------------------------------------------------------------------------

def algorithmic_bytes(seq_lens, H_q, H_kv, d, P, elem, unit, r_kv, kept_tokens, window=False):
    """Bytes per decode-step-layer.

    dense:  every valid K and V row once.
    page:   the page bounds of every page (2 d elements) + K and V of the kept
            pages' valid tokens.
    token:  every valid K row (scoring) + V of the kept tokens.
    window: K and V of the window's tokens (nothing is scored).
    Plus q (read) and out/lse (written, fp32) in every mode.
    kept_tokens: total valid tokens covered by the kept units over all (b, g).
    """
    qo = len(seq_lens) * H_q * (d * elem + d * 4 + 4)
    n_tot = int(np.sum(seq_lens))
    if r_kv >= 1.0:
        return H_kv * n_tot * 2 * d * elem + qo
    if window:
        return kept_tokens * 2 * d * elem + qo
    if unit == "page":
        U_tot = int(np.sum([-(-int(n) // P) for n in seq_lens]))
        return H_kv * U_tot * 2 * d * elem + kept_tokens * 2 * d * elem + qo
    return H_kv * n_tot * d * elem + kept_tokens * d * elem + qo


def attend_bytes(kept_tokens, d, elem, token_unit):
    """Algorithmic bytes of one attention-kernel launch: K and V rows of the
    kept tokens (V only in token unit, where logits are reused); the unit
    scores and q / out are below 0.2% of it and left out."""
    return kept_tokens * (1 if token_unit else 2) * d * elem


def fixed_cost_us(us_sparse, us_dense, b_sparse, b_dense):
    """The sparse step's time beyond its bytes at the dense step's rate:
    us_sparse - us_dense * b_sparse / b_dense ("Where Activation Sparsity and
    KV-Cache Sparsity Cross in LLM Decoding", list view, Table 10: the
    selection's cost beyond byte time).  Positive: fixed costs (launches,
    selection, latency chains) the byte account does not see."""
    return us_sparse - us_dense * b_sparse / b_dense


def kept_token_count(sel, cnt, seq_lens, unit, P):
    total = 0
    for b in range(sel.shape[0]):
        n = int(seq_lens[b])
        for g in range(sel.shape[1]):
            ids = sel[b, g, :cnt[b, g]]
            if unit == "page":
                total += int(np.sum(np.minimum(P, n - ids.astype(np.int64) * P)))
            else:
                total += ids.size
    return total


# ----------------------------------------------------------------------------
# HBM traffic of the dominant kernel from committed rocprofv3 counter passes
# ----------------------------------------------------------------------------

KERNEL_SOURCES = ["attend.hip", "score.hip", "topk.h", "msel.h", "device.h", "kernels.h"]
COPY_BYTES = 1 << 30            # one plain copy: 1 GiB read + 1 GiB written


def kernel_sources_sha():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "sparse_kv_cache_sd_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_file(workload):
    return os.path.join(ROOT, "profiles", f"decode_step_{workload}_traffic.txt")


def read_traffic(workload, tag="attend"):
    """HBM bytes per launch of one kernel of the workload's step ("attend":
    the attention kernel as the step runs it; "score", "dense", "merge"):
    FETCH_SIZE and WRITE_SIZE (KiB per dispatch, rocprofv3 --pmc, one pass
    each) scaled by what the same counters read for a plain 1 GiB copy.
    None when no summary exists, it lacks the kernel, or the kernel sources
    changed since the counters were taken."""
    path = traffic_file(workload)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if "=" in line and not line.lstrip().startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_sources_sha256_16") != kernel_sources_sha():
        return None
    if f"{tag}_fetch_kib_per_dispatch" not in kv:
        return None
    f = float(kv[f"{tag}_fetch_kib_per_dispatch"]) * 1024 * float(kv["fetch_scale"])
    w = float(kv[f"{tag}_write_kib_per_dispatch"]) * 1024 * float(kv["write_scale"])
    return int(f + w)


# the kernels a traffic summary covers, by workload unit: (tag, name pattern)
PMC_KERNELS = {
    "page": [("attend", r"attend_mfma_kernel<\d+, \d+, false, (4|8|32), 0(, \d+)?>"),
             ("score", r"score_pages(_mfma)?_kernel<"),
             ("dense", r"attend_mfma_kernel<\d+, \d+, false, 0, 0(, \d+)?>"),
             ("merge", r"merge_splits_kernel<")],
    "token": [("attend", r"attend_mfma_kernel<\d+, \d+, true, 0, 0(, \d+)?>"),
              ("step_attend", r"attend_mfma_kernel<\d+, \d+, true, 1, 0(, \d+)?>"),
              ("score", r"score_tokens_(mfma|f32)_kernel<"),
              ("dense", r"attend_mfma_kernel<\d+, \d+, false, 0, 0(, \d+)?>"),
              ("merge", r"merge_splits_kernel<")],
}


def copy_calibration():
    """A plain device copy of COPY_BYTES, run a few times, so a counter pass
    over this process also sees what the counters read for known traffic."""
    import torch
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()


def summarize_pmc(fetch_dir, write_dir, workload, out_path, cmd_fetch, cmd_write):
    """Writes the traffic summary from the counter_collection.csv files of
    the two passes: for each kernel of PMC_KERNELS[unit] its mean FETCH_SIZE
    and WRITE_SIZE per dispatch, and the scales from the plain copy."""
    import csv
    import glob
    import re

    def rows(d):
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        assert files, f"no counter_collection.csv under {d}"
        out = []
        for f in files:
            with open(f) as fh:
                out += [(r["Kernel_Name"], r["Dispatch_Id"], float(r["Counter_Value"]))
                        for r in csv.DictReader(fh)]
        return out

    def mean(rs, pred):
        v = [x for n, did, x in rs if pred(n, did)]
        return (sum(v) / len(v), len(v)) if v else (None, 0)

    fr, wr = rows(fetch_dir), rows(write_dir)
    unit = WORKLOADS[workload][2] if workload in WORKLOADS else "page"
    # the plain copy (--copy-calibrate): the blit dispatches that write exactly
    # COPY_BYTES; the fetch pass runs the same program, so the same dispatch
    # ids are the copy there (other device copies, e.g. of layer caches, write
    # other amounts)
    copy_ids = {did for n, did, x in wr
                if "copyBuffer" in n and abs(x - COPY_BYTES / 1024) < 1.0}
    assert copy_ids, "the calibration copy is not in the write pass"
    cp = lambda n, did: "copyBuffer" in n and did in copy_ids
    cf, nf = mean(fr, cp)
    cw, _ = mean(wr, cp)
    assert nf == len(copy_ids), "the fetch pass's dispatch ids differ from the write pass's"
    lines = [
        f"# HBM traffic of the decode step's kernels, workload {workload}",
        "# FETCH_SIZE / WRITE_SIZE are KiB per dispatch (rocprofv3 --pmc, one counter per pass);",
        f"# the scales make a plain {COPY_BYTES} B device copy read and write exactly that.",
        f"# fetch pass: {cmd_fetch}",
        f"# write pass: {cmd_write}",
        f"kernel_sources_sha256_16 = {kernel_sources_sha()}",
        f"copy_bytes = {COPY_BYTES}",
        f"copy_fetch_kib_per_dispatch = {cf:.1f}",
        f"copy_write_kib_per_dispatch = {cw:.1f}",
        f"fetch_scale = {COPY_BYTES / (cf * 1024):.4f}",
        f"write_scale = {COPY_BYTES / (cw * 1024):.4f}",
    ]
    found = 0
    for tag, pat in PMC_KERNELS[unit]:
        rx = re.compile(pat)
        pred = lambda n, gsz, rx=rx: rx.search(n) is not None
        af, an = mean(fr, pred)
        aw, _ = mean(wr, pred)
        if af is None or aw is None:
            continue
        names = sorted({n for n, _, _ in fr if pred(n, None)})
        found += 1
        lines += [f"# {tag}: {names[0][:120]}",
                  f"{tag}_dispatches = {an}",
                  f"{tag}_fetch_kib_per_dispatch = {af:.1f}",
                  f"{tag}_write_kib_per_dispatch = {aw:.1f}"]
    assert found, "none of the step's kernels is in the counter passes"
    with open(out_path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


# ----------------------------------------------------------------------------
# CPU baseline: the oracle, as it stands, on a bounded sample
# ----------------------------------------------------------------------------

def sdref_selection(sel):
    from oracle import sdref
    return sdref.Selection(sel.kind, sel.r_kv, sel.init_units, sel.local_units, sel.max_dropped)


def algorithmic_stats_bytes(seq_lens, H_kv, d, P, elem, scorer):
    """Page statistics read by the scorer: 2 d elements per page (bounds) or
    d fp32 per 16-token window (compressed keys)."""
    if scorer == "compressed":
        return H_kv * int(np.sum([-(-int(n) // 16) for n in seq_lens])) * d * 4
    return H_kv * int(np.sum([-(-int(n) // P) for n in seq_lens])) * 2 * d * elem


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return int(max([p.get("num_threads", 1) for p in threadpool_info()] or [1]))
    except Exception:
        return 1


def oracle_instance(w, b, g):
    """fp64 q of the group and the valid K, V of (sequence b, KV head g)."""
    from oracle import sdref
    r = w.recipe
    G, n = r.group, int(w.seq_lens[b])
    return (sdref.widen(w.q[b, g * G:(g + 1) * G], r.dtype),
            sdref.widen(w.K[b, g, :n], r.dtype), sdref.widen(w.V[b, g, :n], r.dtype))


def oracle_sparse_step(qg, Kg, Vg, stats, unit, P, r_kv, scale):
    """One (sequence, KV head) of the sparse decode step through the oracle's
    own functions: unit scores (from the page bounds, which are setup, or
    from the exact logits), keep count, top-k, softmax over the kept tokens.
    In page unit only the kept pages' keys enter a logit."""
    from oracle import sdref
    n = Kg.shape[0]
    if unit == "page":
        sigma = sdref.page_scores(qg, stats[0], stats[1], scale)
        kept, _ = sdref.select_topk(sigma, sdref.keep_count(r_kv, sigma.shape[0]))
        tokens = sdref.unit_tokens(kept, unit, P, n)
        s = sdref.group_logits(qg, Kg[tokens], scale)
        Vt = Vg[tokens]
        return [sdref.attention(s[i], Vt) for i in range(s.shape[0])]
    s = sdref.group_logits(qg, Kg, scale)
    sigma = sdref.token_scores(s)
    kept, _ = sdref.select_topk(sigma, sdref.keep_count(r_kv, sigma.shape[0]))
    tokens = sdref.unit_tokens(kept, unit, P, n)
    return [sdref.attention(s[i], Vg, tokens) for i in range(s.shape[0])]


def oracle_dense_step(qg, Kg, Vg, scale):
    from oracle import sdref
    s = sdref.group_logits(qg, Kg, scale)
    return [sdref.attention(s[i], Vg) for i in range(s.shape[0])]


def _timed_rounds(fn, n_inst, budget_s, max_rounds):
    """Mean seconds per call of fn(i) over round-robin calls until budget_s
    has passed (at least one call, at most max_rounds passes)."""
    t0 = time.perf_counter()
    done = 0
    while True:
        fn(done % n_inst)
        done += 1
        el = time.perf_counter() - t0
        if el >= budget_s or done >= max_rounds * n_inst:
            return el / done, done, el


def cpu_baseline(w, unit, r_kv, budget_s=12.0, selection=None, scorer="bounds", alpha=None,
                 one_thread=True):
    """The fp64 oracle timed on the host cores over a bounded sample of the
    workload's (sequence, KV head) instances, scaled to microseconds per
    decode-step-layer.  The plain top-k softmax step reports the sparse step
    (value), the dense step and, at one thread, the sparse step again, plus
    the dropped mass delta of the sampled instances; other kept sets and
    alpha-entmax time the oracle's group step (dense and sparse together)."""
    from oracle import entmaxref, sdref
    r = w.recipe
    scale = 1.0 / math.sqrt(r.head_dim)
    groups = [(b, g) for b in range(r.batch) for g in range(r.num_kv_heads)]
    cores = blas_threads()
    base = {"unit": "us/step-layer", "cores": cores, "kind": "oracle", "cpu_model": cpu_model()}
    n_inst = len(groups)
    if selection is not None or alpha is not None or scorer != "bounds":
        def step(i):
            b, g = groups[i]
            qg, Kg, Vg = oracle_instance(w, b, g)
            if alpha is None:
                sdref.group_step(qg, Kg, Vg, unit=unit, page_size=r.page_size, r_kv=r_kv,
                                 scale=scale, selection=selection, scorer=scorer)
            else:
                entmaxref.group_step(qg, Kg, Vg, unit=unit, page_size=r.page_size, r_kv=r_kv,
                                     scale=scale, alpha=alpha, selection=selection, scorer=scorer)
        per, done, el = _timed_rounds(step, n_inst, budget_s, 10 ** 6)
        return dict(base, value=round(per * n_inst * 1e6, 1), sample=(
            f"{done} calls over the step's {n_inst} (sequence, KV head) instances through "
            f"{'oracle.sdref' if alpha is None else 'oracle.entmaxref'}.group_step (fp64 numpy: "
            f"scores, kept set, dense + sparse "
            f"{'softmax' if alpha is None else f'{alpha:g}-entmax'} attention, delta) in "
            f"{el:.1f} s; value = mean time per instance x {n_inst}"))
    # the setup (page bounds) and the fp64 copies of the inputs are made
    # outside the timed calls, as the GPU's page bounds are built beforehand
    # and its inputs are resident before timing
    sample = groups if n_inst <= 16 else groups[:: max(1, n_inst // 16)]
    inst = []
    for b, g in sample:
        qg, Kg, Vg = oracle_instance(w, b, g)
        stats = sdref.page_bounds(Kg, r.page_size) if unit == "page" else None
        inst.append((qg, Kg, Vg, stats))
    m = len(inst)
    sparse = lambda i: oracle_sparse_step(*inst[i][:3], inst[i][3], unit, r.page_size, r_kv, scale)
    dense = lambda i: oracle_dense_step(*inst[i][:3], scale)
    t_sp, n_sp, e_sp = _timed_rounds(sparse, m, 0.4 * budget_s, 10 ** 6)
    t_de, n_de, e_de = _timed_rounds(dense, m, 0.25 * budget_s, 10 ** 6)
    out = dict(base, value=round(t_sp * n_inst * 1e6, 1),
               dense_us_per_step_layer=round(t_de * n_inst * 1e6, 1))
    if one_thread:
        try:
            from threadpoolctl import threadpool_limits
            with threadpool_limits(limits=1):
                t1, n1, e1 = _timed_rounds(sparse, m, 0.2 * budget_s, 10 ** 6)
            out["one_thread_us_per_step_layer"] = round(t1 * n_inst * 1e6, 1)
        except Exception as e:                       # threadpoolctl missing: say so
            out["one_thread_us_per_step_layer"] = None
            log(f"one-thread oracle timing skipped: {e}")
    # dropped mass of the sampled instances (the oracle's group step)
    deltas = []
    for qg, Kg, Vg, _ in inst:
        res = sdref.group_step(qg, Kg, Vg, unit=unit, page_size=r.page_size, r_kv=r_kv,
                               scale=scale)
        deltas.extend(res.delta.tolist())
    out["dropped_mass"] = {"mean": round(float(np.mean(deltas)), 5),
                           "max": round(float(np.max(deltas)), 5),
                           "of": f"the oracle's fp64 delta, every query head of the {m} sampled "
                                 f"(sequence, KV head) instances"}
    out["sample"] = (f"{m} of the step's {n_inst} (sequence, KV head) instances of layer 0, "
                     f"round-robin: sparse step (oracle page_scores / token logits, keep_count, "
                     f"select_topk, attention over the kept tokens; page bounds built "
                     f"beforehand) {n_sp} calls in {e_sp:.1f} s, dense step (logits + attention "
                     f"over every token) {n_de} calls in {e_de:.1f} s; value and dense = mean "
                     f"time per instance x {n_inst}")
    return out


# ----------------------------------------------------------------------------
# GPU measurement of one workload
# ----------------------------------------------------------------------------

MALL_SAFE = 4   # Infinity Caches' worth of other data read between two reads of one layer

# the other points of the metric's 32K-1M range, timed after the main workload
POINTS = ["sweep32k-0.2", "sweep128k-0.3", "sweep128k-0.2", "batch", "l70b-128k", "l70b-1m"]


def layers_for(step_bytes):
    """Distinct layer caches so that between two reads of one layer the steps
    read at least MALL_SAFE x the Infinity Cache of other layers' data."""
    return max(2, math.ceil(MALL_SAFE * MALL_BYTES / max(1, step_bytes)) + 1)


class Measure:
    """Timing of one workload on the GPU: layer caches resident in HBM, the
    sparse step, the dense step and the attention kernel alone, each timed
    over exactly `steps` step-layers with HIP events on the launch stream."""

    def __init__(self, torch, sd, stream, graph):
        self.torch, self.sd, self.stream, self.graph = torch, sd, stream, graph

    def timed(self, fn, steps, warmup, L):
        """Microseconds per call of fn(layer) over exactly `steps` calls, layer
        i mod L for call i.  Untimed first: `warmup` calls, then one pass over
        all L layers, so that every timed call reads a layer last read L
        calls earlier."""
        torch, stream = self.torch, self.stream
        with torch.cuda.stream(stream):
            for i in range(warmup):
                fn(i % L)
            torch.cuda.synchronize()
            if self.graph:
                prime = torch.cuda.CUDAGraph()
                with torch.cuda.graph(prime, stream=stream):
                    for i in range(L):
                        fn(i)
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    for i in range(steps):
                        fn(i % L)
                prime.replay()
            else:
                for i in range(L):
                    fn(i)
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            if self.graph:
                g.replay()
            else:
                for i in range(steps):
                    fn(i % L)
            e1.record(stream)
            torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / steps


def measure_workload(name, args, torch, sd, kvsynth, stream, *, selection_kind="topk",
                     scorer="bounds", entmax=False, main=False, w0=None):
    """Times one workload; returns (result dict, the layer-0 workload)."""
    rname, over, unit, r_kv, desc = WORKLOADS[name]
    if main and args.r_kv > 0:
        r_kv = args.r_kv
        desc += f"; r_KV overridden to {r_kv:g}"
    rec = kvsynth.RECIPES[rname].with_(**over)
    P, d, H_q, H_kv = rec.page_size, rec.head_dim, rec.num_q_heads, rec.num_kv_heads
    elem = 2 if rec.dtype == "bf16" else 4
    dt = torch.bfloat16 if rec.dtype == "bf16" else torch.float32
    t_gen = time.perf_counter()
    if w0 is None:
        w0 = kvsynth.generate(rec)

    def dev(a):
        if rec.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
                torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    pc = w0.paged()
    bt_dev = torch.from_numpy(pc.block_table).cuda()
    sl_dev = torch.from_numpy(w0.seq_lens).cuda()
    shape = sd.Shape(rec.batch, H_q, H_kv, d, P, w0.max_pages(), w0.n_alloc, rec.dtype,
                     pc.num_pages)
    lay0 = dict(q=dev(w0.q), k=dev(pc.k_pool), v=dev(pc.v_pool))
    del pc
    if scorer == "compressed":
        lay0["bounds"] = torch.empty(sd.compressed_keys_shape(shape), dtype=torch.float32,
                                     device="cuda")
        sd.update_compressed_keys(shape, lay0["k"], bt_dev, sl_dev, lay0["bounds"])
    else:
        lay0["bounds"] = torch.empty(sd.bounds_shape(shape), dtype=dt, device="cuda")
        sd.update_page_bounds(shape, lay0["k"], bt_dev, sl_dev, lay0["bounds"])
    torch.cuda.synchronize()
    log(f"{name}: layer 0 resident ({time.perf_counter() - t_gen:.1f} s)")

    structured = selection_kind != "topk" or scorer != "bounds"
    local_units = args.local_units or (2048 // P if unit == "page" else 2048)
    uni = selection_kind == "init_local_topk"
    selection = sd.Selection(selection_kind, r_kv, args.init_units if uni else 0,
                             local_units if uni else 0,
                             args.max_dropped if selection_kind == "mass_budget" else 0.0, scorer)
    config_sel = {}
    if structured:
        config_sel = {"selection": selection_kind, "init_units": selection.init_units,
                      "local_units": selection.local_units,
                      "max_dropped": selection.max_dropped, "scorer": scorer}
        desc += f"; kept set: {selection_kind}" + {
            "init_local_topk": f" ({selection.init_units} initial + {selection.local_units} "
                               f"local units + top-k)",
            "window": " (most recent units)",
            "mass_budget": f" (at most {selection.max_dropped:g} of each head's mass dropped, "
                           f"capped at r_KV)",
            "topk": ""}[selection_kind]
        if scorer == "compressed":
            desc += "; pages scored from compressed keys (mean-pooled, kernel 32 stride 16)"
    if entmax:
        desc += f"; {args.alpha:g}-entmax attention over the kept set (dense: every unit)"
    k_max = sd.selection_capacity(selection, shape.units_max(unit))
    dense_sel = sd.Selection("topk", 1.0)
    if entmax:
        ws = sd.alloc_workspace_entmax(shape, unit, selection)
        ws_dense = sd.alloc_workspace_entmax(shape, unit, dense_sel)
        tau = torch.empty((rec.batch, H_q), dtype=torch.float32, device="cuda")
    else:
        ws = sd.alloc_workspace_sel(shape, unit, selection)
        ws_dense = sd.alloc_workspace(shape, unit, 1.0)
    out = torch.empty((rec.batch, H_q, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((rec.batch, H_q), dtype=torch.float32, device="cuda")
    layers = [lay0]
    sels, cnts = [], []

    def new_sel():
        sels.append(torch.empty((rec.batch, H_kv, k_max), dtype=torch.int32, device="cuda"))
        cnts.append(torch.empty((rec.batch, H_kv), dtype=torch.int32, device="cuda"))

    def sparse_step(i):
        lay = layers[i]
        if entmax:
            sd.decode_step_entmax(shape, lay["q"], lay["k"], lay["v"], lay["bounds"], bt_dev,
                                  sl_dev, unit, selection, args.alpha, out, ws, tau=tau,
                                  sel_idx=sels[i], sel_count=cnts[i], stream=stream)
        elif structured:
            sd.decode_step_sel(shape, lay["q"], lay["k"], lay["v"], lay["bounds"], bt_dev, sl_dev,
                               unit, selection, out, lse, ws, sels[i], cnts[i], stream=stream)
        else:
            sd.decode_step(shape, lay["q"], lay["k"], lay["v"], lay["bounds"], bt_dev, sl_dev,
                           unit, r_kv, out, lse, ws, sels[i], cnts[i], stream=stream)

    def dense_step(i):
        lay = layers[i]
        if entmax:
            sd.decode_step_entmax(shape, lay["q"], lay["k"], lay["v"], None, bt_dev, sl_dev,
                                  unit, dense_sel, args.alpha, out, ws_dense, tau=tau,
                                  stream=stream)
        else:
            sd.decode_step(shape, lay["q"], lay["k"], lay["v"], None, bt_dev, sl_dev, unit, 1.0,
                           out, lse, ws_dense, stream=stream)

    # one sparse step on layer 0 gives the bytes a step reads, which size the
    # layer count
    new_sel()
    with torch.cuda.stream(stream):
        sparse_step(0)
    torch.cuda.synchronize()
    kept = kept_token_count(sels[0].cpu().numpy(), cnts[0].cpu().numpy(), w0.seq_lens, unit, P)
    window = selection_kind == "window"
    b_sparse = algorithmic_bytes(w0.seq_lens, H_q, H_kv, d, P, elem, unit, r_kv, kept,
                                 window=window)
    if unit == "page" and scorer == "compressed" and not window:
        b_sparse += (algorithmic_stats_bytes(w0.seq_lens, H_kv, d, P, elem, "compressed") -
                     algorithmic_stats_bytes(w0.seq_lens, H_kv, d, P, elem, "bounds"))
    b_dense = algorithmic_bytes(w0.seq_lens, H_q, H_kv, d, P, elem, unit, 1.0, 0)
    L = args.layers if main and args.layers else layers_for(b_sparse)
    # layers 1 .. L-1: device copies of layer 0 at their own addresses (the
    # same values, so the same selections; only the addresses differ, which
    # is what keeps a layer out of the caches until it is read again)
    for i in range(1, L):
        layers.append({key: t.clone() for key, t in lay0.items()})
        new_sel()
    torch.cuda.synchronize()
    log(f"{name}: {L} layer caches ({L} x {b_sparse / 1e6:.1f} MB read by the sparse step, "
        f"{L} x {b_dense / 1e6:.1f} MB by the dense step)")

    # scores (and token logits) of every layer, for the attention kernel alone
    umax = shape.units_max(unit)
    scores = [torch.empty((rec.batch, H_kv, umax), dtype=torch.float32, device="cuda")
              for _ in range(L)]
    logits = [torch.empty((rec.batch, H_q, shape.max_seq_len), dtype=torch.float32,
                          device="cuda") if unit == "token" else None for _ in range(L)]
    with torch.cuda.stream(stream):
        for i, lay in enumerate(layers):
            sparse_step(i)
            if scorer == "compressed":
                sd.score_compressed(shape, lay["q"], lay["bounds"], sl_dev, scores[i],
                                    stream=stream)
            else:
                sd.score_pages(shape, lay["q"], lay["k"], lay["bounds"], bt_dev, sl_dev, unit,
                               scores[i], logits[i], stream=stream)
    torch.cuda.synchronize()

    def attend_only(i):
        """The split-K attention kernel alone (one launch), as the decode step
        runs it: page unit selects inside the attention kernel; token unit
        attends the stored selection with the stored logits."""
        lay = layers[i]
        if structured:
            sd.attend_partials(shape, lay["q"], lay["k"], lay["v"], bt_dev, sl_dev, unit, ws,
                               sel_idx=sels[i], sel_count=cnts[i],
                               token_logits=logits[i] if not window else None, stream=stream)
        elif unit == "page":
            sd.attend_partials(shape, lay["q"], lay["k"], lay["v"], bt_dev, sl_dev, unit, ws,
                               unit_scores=scores[i], r_kv=r_kv, stream=stream)
        else:
            sd.attend_partials(shape, lay["q"], lay["k"], lay["v"], bt_dev, sl_dev, unit, ws,
                               sel_idx=sels[i], sel_count=cnts[i], token_logits=logits[i],
                               stream=stream)

    M = Measure(torch, sd, stream, not args.no_graph)
    K, W = args.steps, args.warmup
    us_sparse = M.timed(sparse_step, K, W, L)
    log(f"{name}: sparse step {us_sparse:.2f} us/step-layer over {K} steps")
    us_dense = M.timed(dense_step, K, W, L)
    log(f"{name}: dense step  {us_dense:.2f} us/step-layer")
    us_attend = None
    if not entmax:
        us_attend = M.timed(attend_only, K, W, L)
        log(f"{name}: attention kernel alone {us_attend:.2f} us/launch")
    us_eager = None
    if main and M.graph:
        M.graph = False
        us_eager = M.timed(sparse_step, min(K, 400), W, L)
        M.graph = True
        log(f"{name}: sparse step eager {us_eager:.2f} us/step-layer")

    b_attend = attend_bytes(kept, d, elem, unit == "token" and not window)
    if entmax:
        # several launches behind one entry point: the roofline is the step's
        us_attend, b_attend = us_sparse, b_sparse
    gbps = b_sparse / (us_sparse * 1e-6) / 1e9
    gbps_dense = b_dense / (us_dense * 1e-6) / 1e9
    gbps_att = b_attend / (us_attend * 1e-6) / 1e9
    res = {
        "workload": name,
        "desc": desc,
        "shape": {"batch": rec.batch, "num_q_heads": H_q, "num_kv_heads": H_kv, "head_dim": d,
                  "page_size": P, "context": int(w0.seq_lens.max()), "unit": unit,
                  "r_kv": r_kv, "k_per_kv_head": k_max},
        "layer_caches": L,
        "sparse_footprint_bytes": int(L * b_sparse),
        "us_per_step_layer": round(us_sparse, 3),
        "kept_tokens_per_step": int(kept),
        "effective_gbps": round(gbps, 1),
        "pct_hbm_roofline": round(100 * gbps / HBM_PEAK_GBPS, 1),
        "algorithmic_bytes_per_step": int(b_sparse),
        "dense": {"us_per_step_layer": round(us_dense, 3), "effective_gbps": round(gbps_dense, 1),
                  "pct_hbm_roofline": round(100 * gbps_dense / HBM_PEAK_GBPS, 1),
                  "bytes_per_step": int(b_dense)},
        "speedup_vs_dense": round(us_dense / us_sparse, 3),
        "byte_bound_speedup": round(b_dense / b_sparse, 3),
        "fixed_cost_us": round(fixed_cost_us(us_sparse, us_dense, b_sparse, b_dense), 3),
        "attend": {"us_per_launch": round(us_attend, 3), "bytes_per_launch": int(b_attend),
                   "achieved_gbps": round(gbps_att, 1),
                   "frac": round(gbps_att / HBM_PEAK_GBPS, 4)},
        "traffic": None if structured or entmax else read_traffic(name),
        "structured": structured,
        "config_sel": config_sel,
    }
    if us_eager is not None:
        res["eager_us_per_step_layer"] = round(us_eager, 3)
    if unit == "token" and not entmax and shape.max_seq_len <= 262144:
        # dropped dense softmax mass of layer 0's kept lists (token unit: every
        # logit is stored, so the library computes it on the GPU)
        delta = torch.empty((rec.batch, H_q), dtype=torch.float32, device="cuda")
        sd.dropped_mass(shape, sl_dev, bt_dev, logits[0], sels[0], cnts[0], delta, stream=stream)
        torch.cuda.synchronize()
        dl = delta.cpu().numpy()
        res["dropped_mass"] = {"mean": round(float(dl.mean()), 5), "max": round(float(dl.max()), 5),
                               "of": "layer 0, every query head (sd_dropped_mass)"}
    del layers, lay0, scores, logits, sels, cnts, ws, ws_dense
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res, w0


def bounds_update_times(name, args, torch, sd, kvsynth, stream):
    """Microseconds per call of the three forms of the page-statistics
    update on one workload (graph replays of `steps` calls): a full rebuild,
    the listed pages (each sequence's last page) and the append of one token
    per sequence (folded into its page's bounds)."""
    rname, over = WORKLOADS[name][:2]
    rec = kvsynth.RECIPES[rname].with_(**over)
    w = kvsynth.generate(rec)
    pc = w.paged()
    dt = torch.bfloat16 if rec.dtype == "bf16" else torch.float32

    def dev(a):
        if rec.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
                torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    k = dev(pc.k_pool)
    bt = torch.from_numpy(pc.block_table).cuda()
    sl = torch.from_numpy(w.seq_lens).cuda()
    shape = sd.Shape(rec.batch, rec.num_q_heads, rec.num_kv_heads, rec.head_dim, rec.page_size,
                     w.max_pages(), w.n_alloc, rec.dtype, pc.num_pages)
    bounds = torch.empty(sd.bounds_shape(shape), dtype=dt, device="cuda")
    last = [(b, (int(n) - 1) // rec.page_size) for b, n in enumerate(w.seq_lens)]
    pages = torch.tensor(last, dtype=torch.int32).cuda()
    one = torch.ones(rec.batch, dtype=torch.int32, device="cuda")
    M = Measure(torch, sd, stream, not args.no_graph)
    full = lambda i: sd.update_page_bounds(shape, k, bt, sl, bounds, stream=stream)
    listed = lambda i: sd.update_page_bounds(shape, k, bt, sl, bounds, pages=pages, stream=stream)
    append = lambda i: sd.append_page_bounds(shape, k, bt, sl, one, 1, bounds, stream=stream)
    out = {"workload": name, "batch": rec.batch, "num_kv_heads": rec.num_kv_heads,
           "page_size": rec.page_size, "context_max": int(w.seq_lens.max())}
    for key, fn in (("full_rebuild_us", full), ("last_page_list_us", listed),
                    ("append_one_token_us", append)):
        out[key] = round(M.timed(fn, args.steps, args.warmup, 1), 3)
        log(f"bounds update {name}: {key} = {out[key]}")
    return out


def point_summary(res):
    """The compact form of a workload's result for the main line's points."""
    a = res["attend"]
    return {"workload": res["workload"], "desc": res["desc"], "unit": res["shape"]["unit"],
            "r_kv": res["shape"]["r_kv"], "context": res["shape"]["context"],
            "batch": res["shape"]["batch"], "us_per_step_layer": res["us_per_step_layer"],
            "effective_gbps": res["effective_gbps"], "pct_hbm_roofline": res["pct_hbm_roofline"],
            "dense_us_per_step_layer": res["dense"]["us_per_step_layer"],
            "speedup_vs_dense": res["speedup_vs_dense"],
            "byte_bound_speedup": res["byte_bound_speedup"],
            "fixed_cost_us": res["fixed_cost_us"],
            "attend_us": a["us_per_launch"], "attend_frac": a["frac"],
            "attend_traffic_bytes": res["traffic"],
            "attend_traffic_ratio": (round(res["traffic"] / a["bytes_per_launch"], 3)
                                     if res["traffic"] else None),
            "layer_caches": res["layer_caches"],
            "sparse_footprint_bytes": res["sparse_footprint_bytes"],
            **({"dropped_mass": res["dropped_mass"]} if "dropped_mass" in res else {})}


# ----------------------------------------------------------------------------
# fresh-process blocks (the parent never touches the GPU)
# ----------------------------------------------------------------------------

def child_args(argv):
    """A block's arguments: ours without --blocks, and neither the points nor
    the CPU baseline (the parent times the oracle once)."""
    out, skip = [], False
    for a in argv:
        if skip:
            skip = False
            continue
        if a == "--blocks":
            skip = True
            continue
        if a.startswith("--blocks="):
            continue
        out.append(a)
    return out + ["--no-cpu-baseline", "--no-points"]


def run_blocks(args, argv):
    """Runs `args.blocks` fresh child processes of this script one after
    another (each a whole measurement of the main workload, no points, no
    CPU baseline) and pairs the dense and sparse times within each block."""
    import subprocess
    child = [sys.executable, os.path.abspath(__file__), *child_args(argv)]
    runs = []
    for j in range(args.blocks):
        log(f"block {j + 1}/{args.blocks}: {' '.join(child[1:])}")
        r = subprocess.run(child, capture_output=True, text=True, timeout=900)
        sys.stderr.write(r.stderr[-2000:])
        if r.returncode != 0:
            log(f"block {j + 1} failed with status {r.returncode}")
            sys.exit(r.returncode)
        runs.append(json.loads(r.stdout.strip().splitlines()[-1]))
    sp = np.array([x["value"] for x in runs])
    de = np.array([x["dense"]["us_per_step_layer"] for x in runs])
    ratio = de / sp
    rng = np.random.default_rng(0)
    boot = np.median(ratio[rng.integers(0, len(ratio), size=(4000, len(ratio)))], axis=1)
    boot_sp = np.median(sp[rng.integers(0, len(sp), size=(4000, len(sp)))], axis=1)
    result = runs[int(np.argsort(sp)[len(sp) // 2])]
    result["value"] = round(float(np.median(sp)), 3)
    result["ms_per_step"] = round(result["value"] / 1e3, 6)
    result["blocks"] = {
        "n": len(runs),
        "sparse_us": [round(float(x), 3) for x in sp],
        "dense_us": [round(float(x), 3) for x in de],
        "speedup_paired": [round(float(x), 3) for x in ratio],
        "speedup_median": round(float(np.median(ratio)), 3),
        "speedup_interval_95": [round(float(np.percentile(boot, 2.5)), 3),
                                round(float(np.percentile(boot, 97.5)), 3)],
        "sparse_us_interval_95": [round(float(np.percentile(boot_sp, 2.5)), 3),
                                  round(float(np.percentile(boot_sp, 97.5)), 3)],
        "note": "value = median over fresh-process blocks; intervals from resampling the blocks "
                "(median of each resample), the speedup paired within each block",
    }
    return result


# ----------------------------------------------------------------------------
# main
# ----------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=800, help="decode-step-layers timed")
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="l8b", choices=sorted(WORKLOADS))
    ap.add_argument("--layers", type=int, default=0,
                    help="distinct layer caches (0 = enough that 4x the Infinity Cache of other "
                         "layers is read between two reads of one layer)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-points", action="store_true",
                    help="time only the main workload (not the other 32K-1M points)")
    ap.add_argument("--points", default=",".join(POINTS),
                    help="comma-separated workloads timed after the main one")
    ap.add_argument("--blocks", type=int, default=1,
                    help="N > 1: N fresh processes, paired dense/sparse ratios with a "
                         "resampled interval")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead")
    ap.add_argument("--bounds-update", action="store_true",
                    help="time only the page-statistics updates (full, listed last pages, "
                         "append of one token per sequence) on --workload and exit")
    ap.add_argument("--selection", default="topk",
                    choices=["topk", "window", "init_local_topk", "mass_budget"],
                    help="kept set: top-k (default), the KV window, initial + local + top-k, or "
                         "the dropped-mass budget (token unit)")
    ap.add_argument("--scorer", default="bounds", choices=["bounds", "compressed"],
                    help="page scorer: page bounds (default) or compressed keys")
    ap.add_argument("--max-dropped", type=float, default=0.05,
                    help="mass_budget: most dense softmax mass left outside, per head")
    ap.add_argument("--r-kv", type=float, default=0.0,
                    help="keep ratio (0 = the workload's own)")
    ap.add_argument("--init-units", type=int, default=1, help="init_local_topk: first units kept")
    ap.add_argument("--local-units", type=int, default=0,
                    help="init_local_topk: last units kept (0 = 2048 tokens' worth)")
    ap.add_argument("--attention", default="softmax", choices=["softmax", "entmax"],
                    help="attention over the kept set: softmax (default) or alpha-entmax")
    ap.add_argument("--alpha", type=float, default=1.5, help="entmax alpha in (1, 2]")
    ap.add_argument("--copy-calibrate", action="store_true",
                    help="run a plain 1 GiB copy first (for counter passes)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/decode_step_<workload>_traffic.txt from two "
                         "rocprofv3 --pmc passes and exit")
    ap.add_argument("--pmc-commands", nargs=2, default=["?", "?"],
                    help="the two rocprofv3 command lines, recorded in the summary")
    args = ap.parse_args()

    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.workload,
                      traffic_file(args.workload), *args.pmc_commands)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this decode-attention path has no multi-GPU "
              "mode (its (sequence, KV head) instances are independent, so it would shard "
              "by sequence or by KV head with no exchange); use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    structured = args.selection != "topk" or args.scorer != "bounds"
    entmax = args.attention == "entmax"
    if args.bounds_update:
        import torch
        import kvsynth
        import sparse_kv_cache_sd_amd as sd
        assert torch.cuda.is_available(), "bench.py needs a GPU"
        torch.cuda.set_device(0)
        sd.lib()
        print(json.dumps({"bounds_update": bounds_update_times(
            args.workload, args, torch, sd, kvsynth, torch.cuda.Stream())}), flush=True)
        return
    if args.blocks > 1:
        result = run_blocks(args, sys.argv[1:])
        w0 = None
    else:
        import torch
        import kvsynth
        import sparse_kv_cache_sd_amd as sd

        assert torch.cuda.is_available(), "bench.py needs a GPU"
        torch.cuda.set_device(0)
        sd.lib()  # fail loudly if the HIP library is missing
        if args.copy_calibrate:
            copy_calibration()
        stream = torch.cuda.Stream()
        res, w0 = measure_workload(args.workload, args, torch, sd, kvsynth, stream,
                                   selection_kind=args.selection, scorer=args.scorer,
                                   entmax=entmax, main=True)
        result = {
            "metric": METRIC,
            "value": res["us_per_step_layer"],
            "unit": "us/step-layer",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": args.warmup,
            "ms_per_step": round(res["us_per_step_layer"] / 1e3, 6),
            "higher_is_better": False,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": kvsynth.RECIPES[WORKLOADS[args.workload][0]].dtype,
            "data": "synthetic",
            "config": {"workload": res["desc"], **res["shape"],
                       "layer_caches": res["layer_caches"],
                       "sparse_footprint_bytes": res["sparse_footprint_bytes"],
                       "timing": "eager" if args.no_graph else "hip-graph",
                       **res["config_sel"]},
            "kept_tokens_per_step": res["kept_tokens_per_step"],
            "effective_gbps": res["effective_gbps"],
            "pct_hbm_roofline": res["pct_hbm_roofline"],
            "algorithmic_bytes_per_step": res["algorithmic_bytes_per_step"],
            "dense": res["dense"],
            "speedup_vs_dense": res["speedup_vs_dense"],
            "byte_bound_speedup": res["byte_bound_speedup"],
            "fixed_cost_us": res["fixed_cost_us"],
            "roofline": {
                "kernel": ("whole alpha-entmax decode step (sd_decode_step_entmax)" if entmax else
                           "attend_mfma_kernel: split-K attention partials over the stored kept "
                           "lists" if structured else
                           "attend_mfma_kernel: in-kernel top-k + split-K attention partials "
                           "over the kept pages" if res["shape"]["unit"] == "page" else
                           "attend_mfma_kernel: split-K attention partials over the kept tokens "
                           "(stored logits)"),
                "bound": "hbm", "achieved": res["attend"]["achieved_gbps"],
                "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": res["attend"]["frac"],
                "traffic": res["traffic"],
                "us_per_launch": res["attend"]["us_per_launch"],
                "bytes_per_launch": res["attend"]["bytes_per_launch"],
            },
        }
        if "eager_us_per_step_layer" in res:
            result["eager_us_per_step_layer"] = res["eager_us_per_step_layer"]
        if "dropped_mass" in res:
            result["dropped_mass"] = res["dropped_mass"]
        if entmax:
            result["config"].update({"attention": "entmax", "alpha": args.alpha})
        if not args.no_points and not structured and not entmax:
            pts = []
            cache = {}
            for name in [p for p in args.points.split(",") if p and p != args.workload]:
                key = (WORKLOADS[name][0], tuple(sorted(WORKLOADS[name][1].items())))
                pres, wl = measure_workload(name, args, torch, sd, kvsynth, stream,
                                            w0=cache.get(key))
                cache = {key: wl}         # keep one drawn workload (the 128K pair shares it)
                pts.append(point_summary(pres))
            del cache
            result["points"] = pts
    if not args.no_cpu_baseline:
        import kvsynth
        log("timing the CPU oracle on a bounded sample ...")
        if w0 is None:
            rname, over = WORKLOADS[args.workload][:2]
            w0 = kvsynth.generate(kvsynth.RECIPES[rname].with_(**over))
        unit, r_kv = WORKLOADS[args.workload][2], args.r_kv or WORKLOADS[args.workload][3]
        sel = None
        if structured:
            import sparse_kv_cache_sd_amd as sd
            P = w0.recipe.page_size
            sel = sdref_selection(sd.Selection(
                args.selection, r_kv,
                args.init_units if args.selection == "init_local_topk" else 0,
                (args.local_units or (2048 // P if unit == "page" else 2048))
                if args.selection == "init_local_topk" else 0,
                args.max_dropped if args.selection == "mass_budget" else 0.0, args.scorer))
        result["cpu_baseline"] = cpu_baseline(w0, unit, r_kv, selection=sel, scorer=args.scorer,
                                              alpha=args.alpha if entmax else None)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
