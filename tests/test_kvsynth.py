"""The seeded input generator: storage rounding, paging and reproducibility."""

import numpy as np
import torch

import kvsynth


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.0 - 2 ** -8, 0.0, -0.0], np.float32)])
    mine = kvsynth.to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(mine, ref)


def test_generate_is_seeded_and_paging_round_trips():
    rec = kvsynth.RECIPES["batch"].with_(batch=3, seq_len=700, seq_len_min=300, num_q_heads=8, num_kv_heads=2)
    a = kvsynth.generate(rec)
    b = kvsynth.generate(rec)
    np.testing.assert_array_equal(a.K, b.K)
    np.testing.assert_array_equal(a.q, b.q)
    assert a.seq_lens.min() >= 300 and a.seq_lens.max() <= 700
    pc = a.paged()
    P = rec.page_size
    for bb in range(rec.batch):
        n = int(a.seq_lens[bb])
        U = -(-n // P)
        ids = pc.block_table[bb, :U]
        assert np.all(ids >= 0) and np.all(pc.block_table[bb, U:] == -1)
        for g in range(rec.num_kv_heads):
            k_log = pc.k_pool[ids, g].reshape(U * P, -1)[:n]
            v_log = pc.v_pool[ids, g].reshape(U * P, -1)[:n]
            np.testing.assert_array_equal(k_log, a.K[bb, g, :n])
            np.testing.assert_array_equal(v_log, a.V[bb, g, :n])
    allids = np.concatenate([pc.block_table[bb][pc.block_table[bb] >= 0] for bb in range(rec.batch)])
    assert np.array_equal(np.sort(allids), np.arange(pc.num_pages))


def test_planted_pages_recipe():
    rec = kvsynth.l70b_recipe(128 * 1024).with_(seq_len=64 * 300 + 5)
    w = kvsynth.generate(rec)
    U = -(-int(w.seq_lens[0]) // 64)
    for g in range(rec.num_kv_heads):
        pages = w.salient_pages[(0, g)]
        assert pages.size == int(np.ceil(0.01 * U))
        assert w.salient[(0, g)].size == sum(min(64, int(w.seq_lens[0]) - 64 * u) for u in pages)
