"""GPU parity on seeded random shapes: the whole decode step through the C ABI
against the fp64 oracle on combinations the fixed cases do not pair up --
batch, group size, head dim, page size, dtype, unit, keep ratio and ragged
lengths (empty sequences included) drawn together.  Every shape is one the
library accepts; sizes stay where the oracle finishes in seconds."""

import pytest

import kvsynth

from gpu_util import compare_step, random_shapes, upload

pytestmark = pytest.mark.gpu


CASES = random_shapes(20, 2024)


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
