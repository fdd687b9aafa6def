"""Pins of oracle.bytemodel against the numbers printed on the byte-crossover
page ("Where Activation Sparsity and KV-Cache Sparsity Cross in LLM Decoding",
list view: Tables 1, 2, 9, 11, 14, 17; values in tests/golden/).

Each printed value is matched to half a unit of its last printed digit.
"""

import json
import os

import pytest

from oracle import bytemodel as bm

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "cross_list_tables.json")))
DIMS = GOLD["model_dims"]
K = 1024


def _w(model):
    m = DIMS[model]
    return bm.layer_weights(m["d"], m["d_ff"], m["q_dim"], m["kv_dim"])


def _kv(model):
    return bm.kv_per_token(DIMS[model]["kv_dim"])


def _step_dims(model):
    m = DIMS[model]
    return dict(layers=m["layers"], d=m["d"], d_ff=m["d_ff"], q_dim=m["q_dim"],
                kv_dim=m["kv_dim"], vocab=m["vocab"])


@pytest.mark.parametrize("row", GOLD["table1"]["rows"], ids=lambda r: r["model"])
def test_table1_crossover(row):
    t = GOLD["table1"]
    m = DIMS[row["model"]]
    n_all = bm.crossover(_w(row["model"]), _kv(row["model"]), t["r_p"], t["r_kv"]) / K
    n_ff = bm.crossover(bm.ff_weights(m["d"], m["d_ff"]), _kv(row["model"]), t["r_p"], t["r_kv"]) / K
    assert abs(n_all - row["n_star"]) <= 0.05
    assert abs(n_ff - row["n_star_ff"]) <= 0.05


@pytest.mark.parametrize("row", GOLD["table2"]["rows"], ids=lambda r: f'{r["model"]}-{r["r_p"]}-{r["r_kv"]}')
def test_table2_crossover(row):
    n = bm.crossover(_w(row["model"]), _kv(row["model"]), row["r_p"], row["r_kv"]) / K
    assert abs(n - row["n_star"]) <= 0.05


@pytest.mark.parametrize("row", GOLD["table9"]["rows"], ids=lambda r: str(r["context"]))
def test_table9_accounting(row):
    t = GOLD["table9"]
    parts = bm.step_parts(row["context"], width=t["width"], **_step_dims(t["model"]))
    total = sum(parts.values())
    for key in ("mlp", "attn", "kv", "other"):
        assert abs(100.0 * parts[key] / total - row[key]) <= 0.05, key
    assert abs((1 - t["ff_keep"]) * parts["mlp"] / 1e6 - row["saved_mlp"]) <= 0.5
    assert abs((1 - t["kv_keep"]) * parts["kv"] / 1e6 - row["saved_kv"]) <= 0.5


@pytest.mark.parametrize("row", GOLD["table11"]["rows"], ids=lambda r: str(r["context"]))
def test_table11_window_bound(row):
    t = GOLD["table11"]
    b = bm.byte_bound(row["context"], r_kv=t["r_kv"], **_step_dims(t["model"]))
    assert abs(b - row["bound"]) <= 0.005


@pytest.mark.parametrize("row", GOLD["table17"]["rows"], ids=lambda r: f'{r["r_p"]}-{r["r_kv"]}')
def test_table17_bound(row):
    t = GOLD["table17"]
    b = bm.byte_bound(t["context"], r_p=row["r_p"], r_kv=row["r_kv"], **_step_dims(t["model"]))
    assert abs(b - row["bound"]) <= 0.0005


@pytest.mark.parametrize("row", GOLD["table14"]["rows"], ids=lambda r: str(r["batch"]))
def test_table14_batched_crossover(row):
    """u_B is printed to 2-3 digits, so the crossover is pinned to the interval
    that the rounding of u_B allows, widened by the rounding of n*_B itself."""
    t = GOLD["table14"]
    u = row["union"]
    half = 0.5 * 10.0 ** -(len(u.split(".")[1]))
    lo = bm.batched_crossover(_w(t["model"]), _kv(t["model"]), float(u) + half, row["batch"], t["r_kv"]) / K
    hi = bm.batched_crossover(_w(t["model"]), _kv(t["model"]), float(u) - half, row["batch"], t["r_kv"]) / K
    if "n_star_below" in row:
        assert hi < row["n_star_below"]
        return
    printed = row["n_star"]
    digits = len(str(printed).split(".")[1]) if "." in str(printed) else 0
    pr = 0.5 * 10.0 ** -digits
    assert lo - pr <= printed <= hi + pr


def test_dense_8b_step_at_32k():
    """Dense Llama-3.1-8B step at 32K in BF16: a fixed byte count that the
    Table 11 and 17 bounds are built on (weights 13.96 GB + head 1.05 GB +
    KV 4.29 GB)."""
    b = bm.step_bytes(32768, **_step_dims("Llama-3.1-8B"))
    assert b == 19_304_284_160
