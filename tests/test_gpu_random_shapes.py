"""GPU parity on seeded random shapes: the whole decode step through the C ABI
against the fp64 oracle on combinations the fixed cases do not pair up --
batch, group size, head dim, page size, dtype, unit, keep ratio and ragged
lengths (empty sequences included) drawn together.  Every shape is one the
library accepts; sizes stay where the oracle finishes in seconds."""

import numpy as np
import pytest

import kvsynth

from gpu_util import compare_step, upload

pytestmark = pytest.mark.gpu


def _shapes(n, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        G = int(rng.choice([1, 2, 4, 8]))
        Hkv = int(rng.choice([1, 2, 4, 8]))
        d = int(rng.choice([64, 128]))
        P = int(rng.choice([16, 64]))
        dtype = "f32" if rng.random() < 0.25 else "bf16"
        B = int(rng.integers(1, 5))
        unit = "token" if rng.random() < 0.5 else "page"
        # lengths: mostly short, some past the one-block selection (16384
        # units), some empty
        n_max = int(rng.choice([300, 2000, 9000, 20000, 36000]))
        n_min = int(rng.integers(0, n_max + 1)) if B > 1 else n_max
        r = float(rng.choice([0.02, 0.1, 0.3, 0.5, 0.9, 1.0]))
        empty = B > 1 and rng.random() < 0.3  # the last sequence emptied
        out.append((f"{i:02d}-B{B}-G{G}-H{Hkv}-d{d}-P{P}-{dtype}-{unit}-n{n_max}-r{r}"
                    + ("-empty" if empty else ""),
                    dict(batch=B, num_q_heads=G * Hkv, num_kv_heads=Hkv, head_dim=d,
                         page_size=P, dtype=dtype, seq_len=n_max, seq_len_min=n_min,
                         seed=100 + i), unit, r, empty))
    return out


CASES = _shapes(20)


@pytest.mark.parametrize("cid,kw,unit,r,empty", CASES, ids=[c[0] for c in CASES])
def test_random_shape_decode_step(cid, kw, unit, r, empty):
    print(f"[random-shape] {cid}", flush=True)
    rec = kvsynth.RECIPES["batch"].with_(**kw)
    w = kvsynth.generate(rec)
    dev = upload(w)
    if empty:  # its pages stay allocated; the oracle and the library both see length 0
        w.seq_lens[-1] = 0
        dev.sl[-1] = 0
    compare_step(dev, unit, r)
