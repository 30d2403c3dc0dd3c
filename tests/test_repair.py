"""The margin repairs used by the GPU parity tests (CPU only).

A repair chooses test inputs: it moves two router (or LM-head) columns apart
by whole bf16 steps until every routing (greedy) decision of the oracle's run
has a margin of at least the target. These tests check that a repaired run
really has those margins, that the matrices moved only where and as far as a
repair may move them, and that the run with repaired matrices is an ordinary
oracle run (the hooks choose weights; the arithmetic is unchanged).
"""
import numpy as np

from mkinputs import configs, gen
from oracle import decode as od
from oracle import trajectory as tj
from tests.harness import lm_repair_hook, router_repair_hook

GAP = 2e-2


def _case(B=6, steps=4, seed=5):
    cfg = configs.TINY
    wl = configs.Workload("tiny_rep", cfg, batch=B, seq_len=(10, 60), ragged=True, seed_batch=seed)
    bs = gen.make_batch(wl, extra_steps=steps)
    weights = gen.make_weights(cfg, seed=2, device="cpu")
    pool = gen.bf16_bits(gen.make_kv_pool(cfg, bs.n_pages, seed=seed + 1))
    return cfg, bs, weights, pool


def test_repaired_run_has_the_margins_and_moves_only_whole_steps():
    cfg, bs, weights, pool = _case()
    W = gen.NumpyWeights(weights)
    rh, rrep = router_repair_hook(cfg, gap=GAP)
    lh, lst = lm_repair_hook(gap=GAP)
    bt = bs.block_tables.numpy()
    lens = bs.seq_lens.numpy().astype(np.int64)
    run = tj.greedy_decode(cfg, W, pool.copy(), bt, bs.tokens.numpy(), lens, 4, router_hook=rh, lm_hook=lh)
    # without repairs this draw has small margins (the test exercises repairs)
    plain = tj.greedy_decode(cfg, W, pool.copy(), bt, bs.tokens.numpy(), lens, 4)
    assert min(plain.min_router_gap(cfg.top_k), plain.min_greedy_gap()) < GAP
    assert rrep and lst["wlm"] is not None
    # the repaired matrices differ from the drawn ones in whole bf16 steps, on
    # few columns
    for l, wr in rrep.items():
        a = od.bf16_to_float(W("wr", l), np.float64)
        b = od.bf16_to_float(wr, np.float64)
        cols = np.nonzero(np.any(a != b, axis=0))[0]
        assert 0 < len(cols) <= cfg.n_experts
        d = np.abs(a - b)
        ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(a), 1e-38))) - 7)
        assert np.all(d <= 60 * ulp + 1e-30)
    a = od.bf16_to_float(W("wlm"), np.float64)
    b = od.bf16_to_float(lst["wlm"], np.float64)
    assert 0 < np.count_nonzero(np.any(a != b, axis=0)) <= 2 * lst["repairs"]
    # the recorded run: every step's decisions clear the gap
    assert run.min_router_gap(cfg.top_k) >= GAP * (1 - 1e-4)
    assert run.min_greedy_gap() >= GAP * (1 - 1e-4)


def test_hooks_choose_weights_without_changing_arithmetic():
    """A step with hooks equals a plain step on the matrices the hooks chose."""
    cfg, bs, weights, pool = _case(B=3, seed=9)
    W = gen.NumpyWeights(weights)
    rh, rrep = router_repair_hook(cfg, gap=0.2)   # a wide gap forces repairs
    lh, lst = lm_repair_hook(gap=0.2)
    bt = bs.block_tables.numpy()
    toks, lens = bs.tokens.numpy(), bs.seq_lens.numpy().astype(np.int64)
    lg1, tr1 = od.decode_step(cfg, W, pool.copy(), bt, toks, lens, router_hook=rh, lm_hook=lh)
    assert rrep and lst["wlm"] is not None
    fixed = dict(weights)
    for l, wr in rrep.items():
        fixed[f"wr.{l}"] = gen.torch.from_numpy(wr.view(np.int16).copy()).view(gen.torch.bfloat16)
    fixed["wlm"] = gen.torch.from_numpy(lst["wlm"].view(np.int16).copy()).view(gen.torch.bfloat16)
    lg2, tr2 = od.decode_step(cfg, gen.NumpyWeights(fixed), pool.copy(), bt, toks, lens)
    assert np.array_equal(lg1, lg2)
    for l in range(cfg.n_layers):
        assert np.array_equal(tr1.topk_idx[l], tr2.topk_idx[l])
        assert tj.router_gap(tr2.router_logits[l], cfg.top_k).min() >= 0.2 * (1 - 1e-4)
    assert tj.greedy_gap(lg2).min() >= 0.2 * (1 - 1e-4)
