"""Host logic of bench.py (no GPU): the algorithmic byte model the roofline
divides by, the kept-token count from selections, the traffic summariser
and its staleness check.

The byte model is pinned to the per-configuration figures derived from the
method's byte accounting (all K and V once for dense; page statistics plus
the kept pages' K and V in page unit; all K plus the kept tokens' V in token
unit), computed here from the shapes by hand.
"""

import csv
import os

import numpy as np
import pytest

import bench

K = 1024


def _mb(x):
    return x / 1e6


def test_dense_bytes_8b_32k():
    # 8 KV heads x 32768 tokens x (K + V) x 128 x 2 B, plus q / out / lse
    b = bench.algorithmic_bytes(np.array([32 * K]), 32, 8, 128, 16, 2, "page", 1.0, 0)
    qo = 32 * (128 * 2 + 128 * 4 + 4)
    assert b == 8 * 32 * K * 2 * 128 * 2 + qo
    assert abs(_mb(b) - 134.2) < 0.1


def test_page_bytes_8b_32k():
    # k = 615 of 2048 pages per KV head, all full: 615 * 16 tokens kept per head
    kept = 615 * 16 * 8
    b = bench.algorithmic_bytes(np.array([32 * K]), 32, 8, 128, 16, 2, "page", 0.3, kept)
    meta = 8 * 2048 * 2 * 128 * 2
    kv = kept * 2 * 128 * 2
    assert abs(_mb(meta) - 8.39) < 0.01 and abs(_mb(kv) - 40.30) < 0.01
    assert b == meta + kv + 32 * (128 * 2 + 128 * 4 + 4)
    assert b == 48717952  # the figure the bench line reports at this workload


@pytest.mark.parametrize("n,k,want_mb", [(128 * K, 103, 35.4), (1024 * K, 820, 282.1)])
def test_page_bytes_70b_page64(n, k, want_mb):
    U = n // 64
    kept = k * 64 * 8
    b = bench.algorithmic_bytes(np.array([n]), 64, 8, 128, 64, 2, "page", 0.05, kept)
    assert abs(_mb(b) - want_mb) < 0.1
    assert abs(_mb(8 * U * 2 * 128 * 2) - (8.39 if n == 128 * K else 67.1)) < 0.1


@pytest.mark.parametrize("r,k,want_mb", [(0.3, 39322, 349.0), (0.2, 26215, 322.1)])
def test_token_bytes_8b_128k_token(r, k, want_mb):
    n = 128 * K
    b = bench.algorithmic_bytes(np.array([n]), 32, 8, 128, 16, 2, "token", r, k * 8)
    # every K row once, V of the kept tokens only
    assert b == 8 * n * 128 * 2 + 8 * k * 128 * 2 + 32 * (128 * 2 + 128 * 4 + 4)
    assert abs(_mb(b) - want_mb) < 0.1


def test_window_bytes_read_only_the_window():
    b = bench.algorithmic_bytes(np.array([32 * K]), 32, 8, 128, 16, 2, "page", 0.3, 1000,
                                window=True)
    assert b == 1000 * 2 * 128 * 2 + 32 * (128 * 2 + 128 * 4 + 4)


def test_attend_bytes():
    assert bench.attend_bytes(100, 128, 2, token_unit=False) == 100 * 2 * 128 * 2
    assert bench.attend_bytes(100, 128, 2, token_unit=True) == 100 * 128 * 2


def test_fixed_cost_is_time_beyond_bytes_at_dense_rate():
    # a step that moves a third of the dense bytes in half the dense time
    # spends 50 - 100 / 3 us beyond its byte time
    assert abs(bench.fixed_cost_us(50.0, 100.0, 1.0e6, 3.0e6) - (50.0 - 100.0 / 3)) < 1e-9
    # exactly byte-bound at the dense rate: no fixed cost
    assert bench.fixed_cost_us(25.0, 100.0, 1.0, 4.0) == 0.0


def test_kept_token_count_partial_last_page():
    # one sequence of 40 tokens, pages of 16: pages 0, 1, 2 hold 16, 16, 8 tokens
    sel = np.array([[[0, 2], [1, 2]]], dtype=np.int32)
    cnt = np.array([[2, 1]], dtype=np.int32)
    assert bench.kept_token_count(sel, cnt, np.array([40]), "page", 16) == (16 + 8) + 16
    assert bench.kept_token_count(sel, cnt, np.array([40]), "token", 16) == 3


def _write_pmc(path, rows):
    """rows: dicts with Kernel_Name and Counter_Value; dispatch ids follow the
    order of the list (the same program in both passes)."""
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "pmc_counter_collection.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Dispatch_Id", "Counter_Value"])
        w.writeheader()
        for i, r in enumerate(rows):
            w.writerow({"Kernel_Name": r["Kernel_Name"], "Dispatch_Id": str(i + 1),
                        "Counter_Value": r["Counter_Value"]})


def test_summarize_pmc_picks_the_step_kernels(tmp_path, monkeypatch):
    att = "void sdkv::attend_mfma_kernel<128, 4, false, 4, 0>(sdkv::AttendArgs)"
    dense = "void sdkv::attend_mfma_kernel<128, 4, false, 0, 0>(sdkv::AttendArgs)"
    ent = "void sdkv::attend_mfma_kernel<128, 4, false, 4, 2>(sdkv::AttendArgs)"
    score = "void sdkv::score_pages_kernel<unsigned short, 128, 4>(unsigned short const*)"
    copy = "__amd_rocclr_copyBuffer"
    gib = bench.COPY_BYTES / 1024
    # the same dispatch order in both passes: the 1 GiB calibration copy,
    # a smaller copy (a layer cache), then the step's kernels
    order = [(copy, gib / 2, gib), (copy, 1.0, 8.0), (att, 1000.0, 50.0), (att, 1200.0, 50.0),
             (dense, 9999.0, 70.0), (ent, 7777.0, 1.0), (score, 300.0, 8.0)]
    fetch = [dict(Kernel_Name=n, Counter_Value=f) for n, f, _ in order]
    write = [dict(Kernel_Name=n, Counter_Value=w) for n, _, w in order]
    _write_pmc(str(tmp_path / "f"), fetch)
    _write_pmc(str(tmp_path / "w"), write)
    out = str(tmp_path / "summary.txt")
    bench.summarize_pmc(str(tmp_path / "f"), str(tmp_path / "w"), "l8b", out, "cmd-f", "cmd-w")
    kv = dict(l.split(" = ", 1) for l in open(out).read().splitlines() if " = " in l
              and not l.startswith("#"))
    assert float(kv["attend_fetch_kib_per_dispatch"]) == 1100.0   # mean of the selecting instance
    assert float(kv["attend_write_kib_per_dispatch"]) == 50.0
    assert float(kv["dense_fetch_kib_per_dispatch"]) == 9999.0
    assert float(kv["score_write_kib_per_dispatch"]) == 8.0
    assert "merge_fetch_kib_per_dispatch" not in kv                # not in the passes
    assert abs(float(kv["fetch_scale"]) - 2.0) < 1e-3            # the copy's fetch reads half
    assert abs(float(kv["write_scale"]) - 1.0) < 1e-3
    # the summary is read back only while the kernel sources are unchanged
    monkeypatch.setattr(bench, "traffic_file", lambda wl: out)
    # FETCH and WRITE KiB per dispatch, each scaled by the copy's factor (the
    # scales are stored to four decimals)
    assert abs(bench.read_traffic("l8b") - (1100 * 1024 * 2.0 + 50 * 1024)) < 1024
    assert abs(bench.read_traffic("l8b", "score") - (300 * 1024 * 2.0 + 8 * 1024)) < 1024
    assert bench.read_traffic("l8b", "merge") is None
    stale = str(tmp_path / "stale.txt")
    with open(stale, "w") as fh:
        fh.write(open(out).read().replace(bench.kernel_sources_sha(), "0" * 16))
    monkeypatch.setattr(bench, "traffic_file", lambda wl: stale)
    assert bench.read_traffic("l8b") is None


def test_summarize_pmc_token_attention_instance(tmp_path):
    att = "void sdkv::attend_mfma_kernel<128, 4, true, 0, 0>(sdkv::AttendArgs)"
    sel = "void sdkv::attend_mfma_kernel<128, 4, false, 4, 0>(sdkv::AttendArgs)"
    copy = "__amd_rocclr_copyBuffer"
    gib = bench.COPY_BYTES / 1024
    rows = [dict(Kernel_Name=copy, Counter_Value=gib),
            dict(Kernel_Name=att, Counter_Value=10.0),
            dict(Kernel_Name=sel, Counter_Value=99.0)]
    _write_pmc(str(tmp_path / "f"), rows)
    _write_pmc(str(tmp_path / "w"), rows)
    out = str(tmp_path / "s.txt")
    bench.summarize_pmc(str(tmp_path / "f"), str(tmp_path / "w"), "sweep128k-0.3", out, "f", "w")
    kv = dict(l.split(" = ", 1) for l in open(out).read().splitlines() if " = " in l
              and not l.startswith("#"))
    assert float(kv["attend_fetch_kib_per_dispatch"]) == 10.0


def test_gpus_other_than_one_are_refused():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


@pytest.mark.parametrize("step_mb", [35.4, 48.7, 80.6, 282.1, 349.0, 1021.6, 5000.0])
def test_layer_count_keeps_a_layer_out_of_the_infinity_cache(step_mb):
    """Between two reads of one layer the other L - 1 layers' sparse steps
    read at least 4x the 256 MiB Infinity Cache."""
    b = int(step_mb * 1e6)
    L = bench.layers_for(b)
    assert L >= 2 and (L - 1) * b >= 4 * bench.MALL_BYTES
    assert (L - 2) * b < 4 * bench.MALL_BYTES or L == 2


def test_block_children_drop_blocks_and_extras():
    argv = ["--steps", "20", "--blocks", "5", "--workload", "l8b", "--blocks=3"]
    assert bench.child_args(argv) == ["--steps", "20", "--workload", "l8b",
                                      "--no-cpu-baseline", "--no-points"]
