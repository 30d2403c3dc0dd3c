"""The seeded input generator: determinism, independence, distributions, page tables."""
import json
import os

import numpy as np
import torch

from mkinputs import configs, gen

HERE = os.path.dirname(os.path.abspath(__file__))


def test_weights_deterministic_and_independent():
    cfg = configs.TINY
    a = gen.make_weights(cfg, seed=5)
    b = gen.make_weights(cfg, seed=5)
    c = gen.make_weights(cfg, seed=6)
    for k in a:
        assert a[k].shape == gen.weight_shapes(cfg)[k]
        assert a[k].dtype == torch.bfloat16
        assert torch.equal(a[k].view(torch.int16), b[k].view(torch.int16))
        assert not torch.equal(a[k].view(torch.int16), c[k].view(torch.int16))
    assert not torch.equal(a["wg.0"][0], a["wg.0"][1])
    assert not torch.equal(a["wg.0"], a["wu.0"])


def test_weight_distributions():
    cfg = configs.TINY
    w = gen.make_weights(cfg, seed=7)
    x = w["wg.1"].float()
    assert abs(x.mean().item()) < 1e-3 and abs(x.std().item() - 0.02) < 5e-4
    g = w["gamma.0"].float()
    assert abs(g.mean().item() - 1.0) < 5e-3 and abs(g.std().item() - 0.02) < 5e-3


def test_kv_pool_standard_normal():
    cfg = configs.TINY
    pool = gen.make_kv_pool(cfg, 6, seed=2)
    assert pool.shape == gen.kv_pool_shape(cfg, 6)
    x = pool.float()
    assert abs(x.mean().item()) < 0.02 and abs(x.std().item() - 1.0) < 0.02
    assert not torch.equal(pool[0], pool[1])


def test_batch_page_tables_scattered_and_disjoint():
    wl = configs.Workload("t", configs.FULL48, batch=32, seq_len=(512, 16384), ragged=True)
    bs = gen.make_batch(wl, extra_steps=3)
    lens = bs.seq_lens.numpy()
    assert lens.min() >= 512 and lens.max() <= 16384 and len(set(lens.tolist())) > 20
    bt = bs.block_tables.numpy()
    used = []
    for b in range(32):
        need = -(-(int(lens[b]) + 3) // 16)
        row = bt[b]
        assert np.all(row[:need] >= 0) and np.all(row[need:] == -1)
        used.extend(row[:need].tolist())
    assert len(set(used)) == len(used) == bs.n_pages
    assert sorted(used) != used            # shuffled pool
    bs2 = gen.make_batch(wl, extra_steps=3)
    assert torch.equal(bs.block_tables, bs2.block_tables)


def test_recorded_tiny_seed_still_has_its_margins():
    """The tiny case's recorded seed reproduces the margins the script found."""
    import sys
    sys.path.insert(0, os.path.join(HERE, "golden"))
    import make_tiny_seed as mts
    rec = json.load(open(os.path.join(HERE, "golden", "tiny_seed.json")))
    m = mts.evaluate(rec["seed"])
    assert mts.accepted(m)
    assert m["greedy_tokens"] == rec["greedy_tokens"]
