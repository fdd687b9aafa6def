#!/usr/bin/env python3
"""Decode-attention benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload l8b]
                    [--selection topk|window|init_local_topk|mass_budget]
                    [--scorer bounds|compressed] [--attention softmax|entmax]

A step is one decode step of one attention layer: page-bound (or exact)
scoring, top-k selection under r_KV and split-K attention over the kept
units, merged by log-sum-exp.  Steps cycle over L distinct layer caches whose
total size is at least 4x the 256 MB Infinity Cache, so the KV bytes come from
HBM; the L-layer loop is captured in a HIP graph and replayed.  Inputs are
resident in HBM before timing starts.

Prints ONE JSON line: the metric (microseconds per decode-step-layer, lower
is better), effective HBM GB/s on the algorithmic bytes, the roofline of the
dominant kernel (the split-K attention kernel, timed alone with HIP events on
its stream), the same-kernel dense step for comparison, and the fp64 CPU
oracle timed on a bounded sample on the host cores.  Token-unit lines also
report the dropped softmax mass of layer 0's selection (computed on the GPU).
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

KERNEL_SOURCES = ["attend.hip", "topk.h", "device.h", "kernels.h"]
COPY_BYTES = 1 << 30            # one plain copy: 1 GiB read + 1 GiB written


def kernel_sources_sha():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "sparse_kv_cache_sd_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_file(workload):
    return os.path.join(ROOT, "profiles", f"attend_mfma_{workload}_traffic.txt")


def read_traffic(workload):
    """HBM bytes per launch of the attention kernel: FETCH_SIZE and WRITE_SIZE
    (KiB per dispatch, rocprofv3 --pmc, one pass each) scaled by what the same
    counters read for a plain 1 GiB copy.  None when no summary exists or the
    kernel sources changed since the counters were taken."""
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
    f = float(kv["attend_fetch_kib_per_dispatch"]) * 1024 * float(kv["fetch_scale"])
    w = float(kv["attend_write_kib_per_dispatch"]) * 1024 * float(kv["write_scale"])
    return int(f + w)


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
    the two passes (attention kernel of the page-unit step vs. the copy)."""
    import csv
    import glob

    def rows(d):
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        assert files, f"no counter_collection.csv under {d}"
        out = []
        for f in files:
            with open(f) as fh:
                out += [(r["Kernel_Name"], r["Grid_Size"], float(r["Counter_Value"]))
                        for r in csv.DictReader(fh)]
        return out

    def mean(rs, pred):
        v = [x for n, gsz, x in rs if pred(n, gsz)]
        assert v, "kernel not found in the counter pass"
        return sum(v) / len(v), len(v)

    fr, wr = rows(fetch_dir), rows(write_dir)
    # the in-kernel-selection attention instance: attend_mfma_kernel<D, G,
    # LOGITS = false, SEL in {4, 8, 32}, softmax weights>
    import re
    sel_inst = re.compile(r"attend_mfma_kernel<\d+, \d+, false, (4|8|32), 0>")
    att = lambda n, gsz: sel_inst.search(n) is not None
    af, an = mean(fr, att)
    aw, _ = mean(wr, att)
    # the plain copy: the blit dispatches with the grid of the 1 GiB copy, whose
    # write counter is the largest of the process
    copy_grid = max((x, gsz) for n, gsz, x in wr if "copyBuffer" in n)[1]
    cp = lambda n, gsz: "copyBuffer" in n and gsz == copy_grid
    cf, _ = mean(fr, cp)
    cw, _ = mean(wr, cp)
    anames = [n for n, _, _ in fr if att(n, None)]
    lines = [
        f"# HBM traffic of the in-kernel-selection attention kernel, workload {workload}",
        "# FETCH_SIZE / WRITE_SIZE are KiB per dispatch (rocprofv3 --pmc, one counter per pass);",
        f"# the scales make a plain {COPY_BYTES} B device copy read and write exactly that.",
        f"# fetch pass: {cmd_fetch}",
        f"# write pass: {cmd_write}",
        f"# kernels: {sorted(set(anames))[0][:120]}",
        f"kernel_sources_sha256_16 = {kernel_sources_sha()}",
        f"attend_dispatches = {an}",
        f"attend_fetch_kib_per_dispatch = {af:.1f}",
        f"attend_write_kib_per_dispatch = {aw:.1f}",
        f"copy_bytes = {COPY_BYTES}",
        f"copy_fetch_kib_per_dispatch = {cf:.1f}",
        f"copy_write_kib_per_dispatch = {cw:.1f}",
        f"fetch_scale = {COPY_BYTES / (cf * 1024):.4f}",
        f"write_scale = {COPY_BYTES / (cw * 1024):.4f}",
    ]
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


def cpu_baseline(w, unit, r_kv, budget_s=12.0, selection=None, scorer="bounds", alpha=None):
    from oracle import entmaxref, sdref
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        cores = 1
    r = w.recipe
    G = r.group
    scale = 1.0 / math.sqrt(r.head_dim)
    groups = [(b, g) for b in range(r.batch) for g in range(r.num_kv_heads)]
    t0 = time.perf_counter()
    done = 0
    while True:
        b, g = groups[done % len(groups)]
        n = int(w.seq_lens[b])
        qg = sdref.widen(w.q[b, g * G:(g + 1) * G], r.dtype)
        Kg = sdref.widen(w.K[b, g, :n], r.dtype)
        Vg = sdref.widen(w.V[b, g, :n], r.dtype)
        if alpha is None:
            sdref.group_step(qg, Kg, Vg, unit=unit, page_size=r.page_size, r_kv=r_kv,
                             scale=scale, selection=selection, scorer=scorer)
        else:
            entmaxref.group_step(qg, Kg, Vg, unit=unit, page_size=r.page_size, r_kv=r_kv,
                                 scale=scale, alpha=alpha, selection=selection, scorer=scorer)
        done += 1
        el = time.perf_counter() - t0
        if el >= budget_s or done >= 64 * len(groups):
            break
    per_group = el / done
    us_per_step = per_group * len(groups) * 1e6
    return {"value": round(us_per_step, 1), "unit": "us/step-layer", "cores": int(cores),
            "kind": "oracle",
            "sample": f"{done} runs over the step's {len(groups)} (sequence, KV head) selection "
                      f"instances of layer 0 through "
                      f"{'oracle.sdref' if alpha is None else 'oracle.entmaxref'}.group_step "
                      f"(fp64 numpy: page statistics, scores, top-k, dense + sparse "
                      f"{'softmax' if alpha is None else f'{alpha:g}-entmax'} attention, delta) in "
                      f"{el:.1f} s; value = mean time per instance x {len(groups)}"}


# ----------------------------------------------------------------------------
# main
# ----------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=800, help="decode-step-layers timed")
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="l8b", choices=sorted(WORKLOADS))
    ap.add_argument("--layers", type=int, default=0, help="distinct layer caches (0 = auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead")
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
                    help="write profiles/attend_mfma_<workload>_traffic.txt from two "
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

    import torch
    import kvsynth
    import sparse_kv_cache_sd_amd as sd

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    sd.lib()  # fail loudly if the HIP library is missing
    if args.copy_calibrate:
        copy_calibration()

    rname, over, unit, r_kv, desc = WORKLOADS[args.workload]
    if args.r_kv > 0:
        r_kv = args.r_kv
        desc += f"; r_KV overridden to {r_kv:g}"
    rec = kvsynth.RECIPES[rname].with_(**over)
    P, d, H_q, H_kv = rec.page_size, rec.head_dim, rec.num_q_heads, rec.num_kv_heads
    elem = 2 if rec.dtype == "bf16" else 4

    # ---- layer caches
    w0 = kvsynth.generate(rec)
    dense_layer = H_kv * int(np.sum(w0.seq_lens)) * 2 * d * elem
    L = args.layers or max(1, math.ceil(4 * MALL_BYTES / dense_layer))
    L = min(L, 16)
    log(f"workload {args.workload}: {desc}; {L} layer caches of {dense_layer / 1e6:.1f} MB")
    dt = torch.bfloat16 if rec.dtype == "bf16" else torch.float32

    def dev(a):
        if rec.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    # Every layer has its own K/V pool and query; the sequences' block table
    # and lengths are shared by all layers, as in a serving engine.
    layers = []
    bt_host = None
    for i in range(L):
        w = w0 if i == 0 else kvsynth.generate(rec.with_(seed=rec.seed + 100 * i),
                                               seq_lens=w0.seq_lens)
        pc = w.paged(block_table=bt_host)
        if bt_host is None:
            bt_host = pc.block_table
            bt_dev = torch.from_numpy(bt_host).cuda()
            sl_dev = torch.from_numpy(w0.seq_lens).cuda()
        lay = dict(q=dev(w.q), k=dev(pc.k_pool), v=dev(pc.v_pool), bt=bt_dev, sl=sl_dev,
                   num_pages=pc.num_pages)
        del pc
        if i > 0:
            del w
        layers.append(lay)
        log(f"layer {i} resident")
    num_pages = layers[0]["num_pages"]
    shape = sd.Shape(rec.batch, H_q, H_kv, d, P, w0.max_pages(), w0.n_alloc, rec.dtype, num_pages)
    for lay in layers:
        if args.scorer == "compressed":
            lay["bounds"] = torch.empty(sd.compressed_keys_shape(shape), dtype=torch.float32,
                                        device="cuda")
            sd.update_compressed_keys(shape, lay["k"], lay["bt"], lay["sl"], lay["bounds"])
        else:
            lay["bounds"] = torch.empty(sd.bounds_shape(shape), dtype=dt, device="cuda")
            sd.update_page_bounds(shape, lay["k"], lay["bt"], lay["sl"], lay["bounds"])
    torch.cuda.synchronize()

    structured = args.selection != "topk" or args.scorer != "bounds"
    local_units = args.local_units or (2048 // P if unit == "page" else 2048)
    selection = sd.Selection(args.selection, r_kv,
                             args.init_units if args.selection == "init_local_topk" else 0,
                             local_units if args.selection == "init_local_topk" else 0,
                             args.max_dropped if args.selection == "mass_budget" else 0.0,
                             args.scorer)
    if structured:
        config_sel = {"selection": args.selection, "init_units": selection.init_units,
                      "local_units": selection.local_units,
                      "max_dropped": selection.max_dropped, "scorer": args.scorer}
        desc += f"; kept set: {args.selection}" + {
            "init_local_topk": f" ({selection.init_units} initial + {selection.local_units} "
                               f"local units + top-k)",
            "window": " (most recent units)",
            "mass_budget": f" (at most {selection.max_dropped:g} of each head's mass dropped, "
                           f"capped at r_KV)",
            "topk": ""}[args.selection]
        if args.scorer == "compressed":
            desc += "; pages scored from compressed keys (mean-pooled, kernel 32 stride 16)"
    entmax = args.attention == "entmax"
    if entmax:
        desc += f"; {args.alpha:g}-entmax attention over the kept set (dense: every unit)"
    k_max = sd.selection_capacity(selection, shape.units_max(unit))
    ws = sd.alloc_workspace_sel(shape, unit, selection)
    ws_dense = sd.alloc_workspace(shape, unit, 1.0)
    dense_sel = sd.Selection("topk", 1.0)
    if entmax:
        ws = sd.alloc_workspace_entmax(shape, unit, selection)
        ws_dense = sd.alloc_workspace_entmax(shape, unit, dense_sel)
        tau = torch.empty((rec.batch, H_q), dtype=torch.float32, device="cuda")
    out = torch.empty((rec.batch, H_q, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((rec.batch, H_q), dtype=torch.float32, device="cuda")
    sels = [torch.empty((rec.batch, H_kv, k_max), dtype=torch.int32, device="cuda") for _ in range(L)]
    cnts = [torch.empty((rec.batch, H_kv), dtype=torch.int32, device="cuda") for _ in range(L)]
    stream = torch.cuda.Stream()

    def sparse_step(i):
        lay = layers[i]
        if entmax:
            sd.decode_step_entmax(shape, lay["q"], lay["k"], lay["v"], lay["bounds"], lay["bt"],
                                  lay["sl"], unit, selection, args.alpha, out, ws, tau=tau,
                                  sel_idx=sels[i], sel_count=cnts[i], stream=stream)
        elif structured:
            sd.decode_step_sel(shape, lay["q"], lay["k"], lay["v"], lay["bounds"], lay["bt"],
                               lay["sl"], unit, selection, out, lse, ws, sels[i], cnts[i],
                               stream=stream)
        else:
            sd.decode_step(shape, lay["q"], lay["k"], lay["v"], lay["bounds"], lay["bt"],
                           lay["sl"], unit, r_kv, out, lse, ws, sels[i], cnts[i], stream=stream)

    def dense_step(i):
        lay = layers[i]
        if entmax:
            sd.decode_step_entmax(shape, lay["q"], lay["k"], lay["v"], None, lay["bt"], lay["sl"],
                                  unit, dense_sel, args.alpha, out, ws_dense, tau=tau,
                                  stream=stream)
        else:
            sd.decode_step(shape, lay["q"], lay["k"], lay["v"], None, lay["bt"], lay["sl"],
                           unit, 1.0, out, lse, ws_dense, stream=stream)

    # scores of every layer, for timing the attention stage on its own
    umax = shape.units_max(unit)
    scores = [torch.empty((rec.batch, H_kv, umax), dtype=torch.float32, device="cuda")
              for _ in range(L)]
    logits = [torch.empty((rec.batch, H_q, shape.max_seq_len), dtype=torch.float32, device="cuda")
              if unit == "token" else None for _ in range(L)]
    for i, lay in enumerate(layers):
        if args.scorer == "compressed":
            sd.score_compressed(shape, lay["q"], lay["bounds"], lay["sl"], scores[i], stream=stream)
        else:
            sd.score_pages(shape, lay["q"], lay["k"], lay["bounds"], lay["bt"], lay["sl"], unit,
                           scores[i], logits[i], stream=stream)
    torch.cuda.synchronize()

    def attend_only(i):
        """The split-K attention kernel alone (one launch), as the decode step
        runs it: page unit selects inside the attention kernel; token unit
        attends the stored selection with the stored logits."""
        lay = layers[i]
        if structured:
            sd.attend_partials(shape, lay["q"], lay["k"], lay["v"], lay["bt"], lay["sl"], unit, ws,
                               sel_idx=sels[i], sel_count=cnts[i],
                               token_logits=logits[i] if args.selection != "window" else None,
                               stream=stream)
        elif unit == "page":
            sd.attend_partials(shape, lay["q"], lay["k"], lay["v"], lay["bt"], lay["sl"], unit, ws,
                               unit_scores=scores[i], r_kv=r_kv, stream=stream)
        else:
            sd.attend_partials(shape, lay["q"], lay["k"], lay["v"], lay["bt"], lay["sl"], unit, ws,
                               sel_idx=sels[i], sel_count=cnts[i], token_logits=logits[i],
                               stream=stream)

    def timed(fn, steps, warmup, graph):
        """Mean microseconds per call of fn(layer) over `steps` calls cycling layers."""
        with torch.cuda.stream(stream):
            for i in range(warmup):
                fn(i % L)
            torch.cuda.synchronize()
            reps = max(1, steps // L)
            if graph:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    for i in range(L):
                        fn(i)
                g.replay()
                torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(reps):
                if graph:
                    g.replay()
                else:
                    for i in range(L):
                        fn(i)
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1e3 / (reps * L), reps * L

    graph = not args.no_graph
    # warm selections so attend_only has valid inputs
    with torch.cuda.stream(stream):
        for i in range(L):
            sparse_step(i)
    torch.cuda.synchronize()

    us_sparse, n_steps = timed(sparse_step, args.steps, args.warmup, graph)
    log(f"sparse step: {us_sparse:.2f} us/step-layer over {n_steps} steps ({'graph' if graph else 'eager'})")
    us_dense, _ = timed(dense_step, args.steps, args.warmup, graph)
    log(f"dense step:  {us_dense:.2f} us/step-layer")
    if not entmax:
        us_attend, n_att = timed(attend_only, args.steps, args.warmup, graph)
        log(f"attend alone (HIP events on its stream): {us_attend:.2f} us/launch")
    us_sparse_eager, _ = timed(sparse_step, min(args.steps, 400), 10, False)
    log(f"sparse step eager: {us_sparse_eager:.2f} us/step-layer")

    # bytes from the actual selections
    kept = []
    for i in range(L):
        kept.append(kept_token_count(sels[i].cpu().numpy(), cnts[i].cpu().numpy(),
                                     w0.seq_lens, unit, P))
    kept_mean = float(np.mean(kept))
    window = args.selection == "window"
    b_sparse = algorithmic_bytes(w0.seq_lens, H_q, H_kv, d, P, elem, unit, r_kv, kept_mean,
                                 window=window)
    if unit == "page" and args.scorer == "compressed" and not window:
        b_sparse += (algorithmic_stats_bytes(w0.seq_lens, H_kv, d, P, elem, "compressed") -
                     algorithmic_stats_bytes(w0.seq_lens, H_kv, d, P, elem, "bounds"))
    b_dense = algorithmic_bytes(w0.seq_lens, H_q, H_kv, d, P, elem, unit, 1.0, 0)
    b_attend = attend_bytes(kept_mean, d, elem, unit == "token" and not window)
    gbps = b_sparse / (us_sparse * 1e-6) / 1e9
    gbps_dense = b_dense / (us_dense * 1e-6) / 1e9
    if entmax:
        # The entmax step is several launches (scores, selection, logits of
        # the kept tokens, thresholds, attention, merge) behind one entry
        # point, so the roofline here is that of the whole step on its
        # algorithmic bytes; per-kernel durations come from a kernel trace.
        us_attend, b_attend = us_sparse, b_sparse
    gbps_att = b_attend / (us_attend * 1e-6) / 1e9

    result = {
        "metric": METRIC,
        "value": round(us_sparse, 3),
        "unit": "us/step-layer",
        "n_gpus": 1,
        "steps": n_steps,
        "warmup": args.warmup,
        "ms_per_step": round(us_sparse / 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": rec.dtype,
        "data": "synthetic",
        "config": {
            "workload": desc,
            "batch": rec.batch, "num_q_heads": H_q, "num_kv_heads": H_kv, "head_dim": d,
            "page_size": P, "context": int(w0.seq_lens.max()), "unit": unit, "r_kv": r_kv,
            "k_per_kv_head": k_max, "layer_caches": L, "timing": "hip-graph" if graph else "eager",
        },
        "kept_tokens_per_step": round(kept_mean, 1),
        "effective_gbps": round(gbps, 1),
        "pct_hbm_roofline": round(100 * gbps / HBM_PEAK_GBPS, 1),
        "algorithmic_bytes_per_step": int(b_sparse),
        "dense": {"us_per_step_layer": round(us_dense, 3), "effective_gbps": round(gbps_dense, 1),
                  "pct_hbm_roofline": round(100 * gbps_dense / HBM_PEAK_GBPS, 1),
                  "bytes_per_step": int(b_dense)},
        "speedup_vs_dense": round(us_dense / us_sparse, 3),
        "byte_bound_speedup": round(b_dense / b_sparse, 3),
        "eager_us_per_step_layer": round(us_sparse_eager, 3),
        "roofline": {
            "kernel": ("whole alpha-entmax decode step (sd_decode_step_entmax)" if entmax else
                       "attend_mfma_kernel: split-K attention partials over the stored kept "
                       "lists" if structured else
                       "attend_mfma_kernel: in-kernel top-k + split-K attention partials over "
                       "the kept pages" if unit == "page" else
                       "attend_mfma_kernel: split-K attention partials over the kept tokens "
                       "(stored logits)"),
            "bound": "hbm", "achieved": round(gbps_att, 1), "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": round(gbps_att / HBM_PEAK_GBPS, 4),
            "traffic": (read_traffic(args.workload)
                        if unit == "page" and not structured and not entmax else None),
            "us_per_launch": round(us_attend, 3), "bytes_per_launch": int(b_attend),
        },
    }
    if unit == "token" and not entmax and shape.max_seq_len <= 262144:
        # dropped dense softmax mass of layer 0's kept lists (token unit: every
        # logit is stored, so the library computes it on the GPU)
        delta = torch.empty((rec.batch, H_q), dtype=torch.float32, device="cuda")
        sd.dropped_mass(shape, layers[0]["sl"], layers[0]["bt"], logits[0], sels[0], cnts[0],
                        delta, stream=stream)
        torch.cuda.synchronize()
        dl = delta.cpu().numpy()
        result["dropped_mass"] = {"mean": round(float(dl.mean()), 5),
                                  "max": round(float(dl.max()), 5),
                                  "of": "layer 0, every query head (sd_dropped_mass)"}
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        result["cpu_baseline"] = cpu_baseline(
            w0, unit, r_kv, selection=None if not structured else sdref_selection(selection),
            scorer=args.scorer, alpha=args.alpha if entmax else None)
    if structured:
        result["config"].update(config_sel)
    if entmax:
        result["config"].update({"attention": "entmax", "alpha": args.alpha})
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
