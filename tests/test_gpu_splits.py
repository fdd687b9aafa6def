"""Split-K partition invariance on the GPU, through sd_attend_splitk.

The split plan cuts each (sequence, KV head)'s kept list into splits of
E = ceil(k_max / S) entries, S fixed by the machine, so the same kept list
stored in rows of different length k_max is attended under different
partitions: the split boundaries move, and once k_max exceeds a row's count
the later splits hold nothing (empty splits, lse = -inf).  The pages leave
the partition free ([Cross/list] Abstract: dense and sparse decoding through
one split-K kernel; the log-sum-exp merge makes the result independent of
it), so every run must match the fp64 oracle on the same kept set, and the
runs must agree with each other far more tightly than that tolerance.
"""

import math

import numpy as np
import pytest
import torch

import kvsynth
import sparse_kv_cache_sd_amd as sd

from gpu_util import TOL, oracle_group, upload

pytestmark = pytest.mark.gpu

R = kvsynth.RECIPES

# agreement between partitions: fp32 accumulation in another order (bf16
# weights are carried as a bf16 hi + lo pair, about 16 significant bits)
MUTUAL = {"f32": 2e-6, "bf16": 2e-4}

CASES = [
    ("l8b", dict(seq_len=5000, num_q_heads=16, num_kv_heads=4), "page", 0.3, True),
    ("batch", dict(batch=3, seq_len=3000, seq_len_min=200, num_q_heads=16, num_kv_heads=4),
     "page", 0.2, True),
    ("l70b", dict(seq_len=64 * 40 + 5), "page", 0.05, True),
    ("sweep", dict(seq_len=3000, num_q_heads=16, num_kv_heads=4), "token", 0.3, True),
    ("sweep", dict(seq_len=3000, num_q_heads=16, num_kv_heads=4), "token", 0.3, False),
    ("tiny", dict(), "token", 0.25, True),
    ("tiny", dict(), "token", 0.25, False),
]


@pytest.mark.parametrize("name,kw,unit,r,use_logits", CASES,
                         ids=[f"{c[0]}-{c[2]}-{c[3]}-{'logits' if c[4] else 'qk'}" for c in CASES])
def test_split_partition_invariance(name, kw, unit, r, use_logits):
    w = kvsynth.generate(R[name].with_(**kw))
    dev = upload(w)
    s = dev.shape
    scale = 1 / math.sqrt(s.head_dim)
    umax = s.units_max(unit)
    orcs = {(b, g): oracle_group(w, b, g, unit, r, scale)
            for b in range(s.batch) for g in range(s.num_kv_heads)}
    k0 = max(o.k for o in orcs.values())
    logits = None
    if unit == "token" and use_logits:
        scores = torch.empty((s.batch, s.num_kv_heads, umax), dtype=torch.float32, device="cuda")
        logits = torch.empty((s.batch, s.num_q_heads, s.max_seq_len), dtype=torch.float32,
                             device="cuda")
        sd.score_pages(s, dev.q, dev.k, dev.bounds, dev.bt, dev.sl, unit, scores, logits)
    ws = sd.alloc_workspace(s, unit, 1.0)
    G, tol = s.group, TOL[s.dtype]
    row_lengths = sorted({k0, min(umax, k0 + 37), min(umax, 2 * k0 + 5), umax})
    assert len(row_lengths) >= 3
    runs = []
    for k_max in row_lengths:
        # entries past a row's count hold unit 0: read by mistake, it would
        # count a token twice and move the output
        sel = np.zeros((s.batch, s.num_kv_heads, k_max), dtype=np.int32)
        cnt = np.zeros((s.batch, s.num_kv_heads), dtype=np.int32)
        for (b, g), o in orcs.items():
            sel[b, g, :o.k] = o.kept
            cnt[b, g] = o.k
        out = torch.full((s.batch, s.num_q_heads, s.head_dim), float("nan"), device="cuda")
        lse = torch.full((s.batch, s.num_q_heads), float("nan"), device="cuda")
        sd.attend_splitk(s, dev.q, dev.k, dev.v, dev.bt, dev.sl, unit,
                         torch.from_numpy(sel).cuda(), torch.from_numpy(cnt).cuda(), out, lse, ws,
                         token_logits=logits)
        torch.cuda.synchronize()
        out, lse = out.cpu().numpy(), lse.cpu().numpy()
        for (b, g), o in orcs.items():
            hs = slice(g * G, (g + 1) * G)
            e_o = np.abs(out[b, hs] - o.out_sparse).max()
            e_l = np.abs(lse[b, hs] - o.lse_sparse).max()
            assert e_o <= tol and e_l <= tol, f"k_max={k_max} (b={b}, g={g}): {e_o}, {e_l}"
        runs.append((k_max, out, lse))
    worst = 0.0
    for k_max, out, lse in runs[1:]:
        d_o = float(np.abs(out - runs[0][1]).max())
        d_l = float(np.abs(lse - runs[0][2]).max())
        assert d_o <= MUTUAL[s.dtype] and d_l <= MUTUAL[s.dtype], \
            f"row length {k_max} vs {runs[0][0]}: out {d_o}, lse {d_l}"
        worst = max(worst, d_o, d_l)
    print(f"[splits] {name} {unit} r={r}: row lengths {row_lengths}, largest difference "
          f"between partitions {worst:.2e}", flush=True)
