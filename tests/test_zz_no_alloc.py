"""The allocation-free step (mk_decode_step_noalloc) against mk_decode_step.

Two handles decode the same inputs from two copies of one KV cache: one with
mk_decode_step (the handle's scratch), one with mk_decode_step_noalloc (the
device's static scratch array). Two calls in a row, the second with a smaller
batch and shorter contexts, in both modes: logits, greedy tokens and the
appended K/V must be bit-identical (the same kernels and schedule on the same
inputs). Also: a schedule that was never built is refused (building one
allocates), and a model whose step scratch exceeds the static array is
refused with MK_ERR_UNSUPPORTED.
"""
import numpy as np
import pytest
import torch

import moe_persistent_decode_amd as mk
from mkinputs import configs, gen
from tests.harness import bits_to_torch, say, tiny_seed, torch_to_bits

pytestmark = pytest.mark.gpu


def _batch(cfg, B, lo, hi, seed):
    wl = configs.Workload(f"noalloc_b{B}", cfg, batch=B, seq_len=(lo, hi), ragged=True, seed_batch=seed)
    return gen.make_batch(wl, extra_steps=1)


@pytest.mark.parametrize("mode", [0, 1])
def test_noalloc_step_equals_the_allocating_step(mode):
    cfg = configs.TINY_WIN
    big, small = _batch(cfg, 4, 60, 180, 301), _batch(cfg, 2, 10, 40, 302)
    n_pages = max(big.n_pages, small.n_pages)
    mpps = max(big.max_pages_per_seq, small.max_pages_per_seq)
    pool0 = gen.bf16_bits(gen.make_kv_pool(cfg, n_pages, seed=303))
    weights = {k: v.cuda() for k, v in gen.make_weights(cfg, seed=tiny_seed()["seed"]).items()}
    mc = mk.make_config(cfg, 4, mpps * cfg.page_size, n_pages, mpps, mode)
    pools = [bits_to_torch(pool0), bits_to_torch(pool0)]
    decs = [mk.Decoder(mc, p) for p in pools]
    try:
        for d in decs:
            d.load_weights(weights)
        for i, bs in enumerate((big, small)):
            B = bs.tokens.shape[0]
            bt = torch.full((B, mpps), -1, dtype=torch.int32)
            bt[:, :bs.max_pages_per_seq] = bs.block_tables
            bt = bt.cuda()
            hint = int(bs.seq_lens.max())
            out = []
            for k, d in enumerate(decs):
                logits = torch.full((B, cfg.vocab), float("nan"), dtype=torch.float32, device="cuda")
                nxt = torch.full((B,), -1, dtype=torch.int32, device="cuda")
                toks, lens = bs.tokens.cuda(), bs.seq_lens.cuda()
                if k == 0:
                    d.step(toks, bt, lens, hint, logits, nxt)
                else:
                    # a schedule never built for these sizes is refused (building allocates)
                    with pytest.raises(mk.MkError) as e:
                        d.step_noalloc(toks, bt, lens, hint, logits, nxt)
                    assert e.value.status == 7, str(e.value)
                    d.schedule_info(B, hint)  # builds and caches the schedule
                    d.step_noalloc(toks, bt, lens, hint, logits, nxt)
                d.sync()
                out.append((logits.cpu().numpy(), nxt.cpu().numpy()))
            assert np.array_equal(out[0][0], out[1][0]), f"call {i}: logits differ"
            assert np.array_equal(out[0][1], out[1][1]), f"call {i}: tokens differ"
            assert np.array_equal(torch_to_bits(pools[0]), torch_to_bits(pools[1])), f"call {i}: KV differs"
            say(f"[noalloc mode={mode}] call {i} (batch {B}, lengths {int(bs.seq_lens.min())}..{hint}): "
                f"bit-identical to mk_decode_step")
    finally:
        for d in decs:
            d.close()


def test_noalloc_refuses_a_model_beyond_the_static_array():
    # 32 sequences of a 256K context: the attention partials alone exceed 64 MiB
    m = configs.small_variant(configs.FULL48, n_layers=1, vocab=1024)
    mpps = 262144 // 16 + 1
    mc = mk.make_config(m, 32, 262144, 64, mpps, 0)
    d = mk.Decoder(mc, None)
    try:
        w = {k: v.cuda() for k, v in gen.make_weights(m, seed=5).items()}
        d.load_weights(w)
        toks = torch.zeros(32, dtype=torch.int32, device="cuda")
        lens = torch.ones(32, dtype=torch.int32, device="cuda")
        bt = torch.zeros((32, mpps), dtype=torch.int32, device="cuda")
        logits = torch.empty((32, m.vocab), dtype=torch.float32, device="cuda")
        with pytest.raises(mk.MkError) as e:
            d.step_noalloc(toks, bt, lens, 1, logits)
        assert e.value.status == 2, str(e.value)
        say(f"[noalloc] {e.value}")
    finally:
        d.close()
