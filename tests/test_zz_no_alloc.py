"""The allocation-free decode step (sd_decode_step_noalloc, scratch in a
static device array) against sd_decode_step with a caller workspace: the same
kernels on the same inputs, so the kept lists must be identical and the
outputs within the parity tolerances (they are expected bit-identical).

Two calls in a row, the second with a smaller input, show that what the
first call leaves in the shared scratch does not leak into the second.
(The refusal of sizes past the static scratch is a host-side check, tested
without a GPU in test_abi.py.)"""

import numpy as np
import pytest
import torch

import kvsynth
import sparse_kv_cache_sd_amd as sd

from gpu_util import TOL, upload

pytestmark = pytest.mark.gpu

R = kvsynth.RECIPES


def _run(dev, unit, r, noalloc):
    s = dev.shape
    out = torch.full((s.batch, s.num_q_heads, s.head_dim), float("nan"), device="cuda")
    lse = torch.full((s.batch, s.num_q_heads), float("nan"), device="cuda")
    sel = cnt = None
    if r < 1.0:
        k_max = sd.keep_count(r, s.units_max(unit))
        sel = torch.full((s.batch, s.num_kv_heads, k_max), -7, dtype=torch.int32, device="cuda")
        cnt = torch.full((s.batch, s.num_kv_heads), -7, dtype=torch.int32, device="cuda")
    if noalloc:
        sd.decode_step_noalloc(s, dev.q, dev.k, dev.v, dev.bounds, dev.bt, dev.sl, unit, r, out,
                               lse, sel_idx=sel, sel_count=cnt)
    else:
        ws = sd.alloc_workspace(s, unit, r)
        sd.decode_step(s, dev.q, dev.k, dev.v, dev.bounds, dev.bt, dev.sl, unit, r, out, lse, ws,
                       sel_idx=sel, sel_count=cnt)
    torch.cuda.synchronize()
    return (out.cpu().numpy(), lse.cpu().numpy(),
            None if sel is None else sel.cpu().numpy(), None if cnt is None else cnt.cpu().numpy())


def _same(a, b, dtype):
    tol = TOL[dtype]
    assert np.all(np.isfinite(a[0])) and np.all(np.isfinite(a[1]))
    assert np.abs(a[0] - b[0]).max() <= tol and np.abs(a[1] - b[1]).max() <= tol
    if a[2] is not None:
        np.testing.assert_array_equal(a[3], b[3])
        for bb in range(a[3].shape[0]):
            for g in range(a[3].shape[1]):
                k = int(a[3][bb, g])
                np.testing.assert_array_equal(a[2][bb, g, :k], b[2][bb, g, :k])
    return bool(np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]))


# (first call, second call with a smaller input)
PAIRS = [
    (("sweep", dict(seq_len=40000), "token", 0.2),         # many-block top-k, logits in scratch
     ("batch", dict(batch=3, seq_len=5000, seq_len_min=300), "page", 0.3)),
    (("l70b", dict(seq_len=64 * 300 + 17), "page", 0.05),
     ("tiny", dict(), "token", 0.25)),
    (("l8b", dict(seq_len=20000), "page", 1.0),             # dense
     ("l8b", dict(seq_len=3000, num_q_heads=8, num_kv_heads=2), "page", 0.3)),
]


@pytest.mark.parametrize("first,second", PAIRS, ids=[f"{a[0]}-{a[2]}-then-{b[0]}-{b[2]}"
                                                     for a, b in PAIRS])
def test_noalloc_matches_workspace_entry(first, second):
    for name, kw, unit, r in (first, second):
        dev = upload(kvsynth.generate(R[name].with_(**kw)))
        ref = _run(dev, unit, r, noalloc=False)
        got = _run(dev, unit, r, noalloc=True)
        ident = _same(got, ref, dev.shape.dtype)
        again = _run(dev, unit, r, noalloc=True)     # the scratch now holds this call's data
        _same(again, ref, dev.shape.dtype)
        print(f"[noalloc] {name} {unit} r={r}: matches the workspace entry "
              f"({'bit-identical' if ident else 'within tolerance'})", flush=True)

