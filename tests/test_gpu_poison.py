"""GPU: the debug poison mode (mk_set_debug_poison) as a read-before-write
check of the whole schedule.

Before each poisoned step every per-step scratch buffer holds NaN (tagged
words NaN with tag 0, index buffers 0), so a task that read a value before
its producer stored it would carry NaN into the logits, or an impossible
value into the argmax (reported as a device fault). Each case decodes one
step clean and the same step again poisoned, from the same inputs, and
requires bit-identical logits and greedy tokens; a buffer row past the batch
shows that the fill ran. Batches 1 and 4 (fused MoE, tagged hand-offs) and 32
(claiming MoE), the sliding-window tiny model and one full-size layer,
megakernel and kernel-per-op modes, the allocation-free step, and the tiny
dense model (megakernel post,
Chinese version, barrier section: a wrong arrival lets a reader run ahead
and fail later).
"""
import numpy as np
import pytest
import torch

from mkinputs import configs, gen
from tests.harness import bits_to_torch, make_decoder, say, tiny_seed

pytestmark = pytest.mark.gpu


def _steps(cfg, B, mode, noalloc=False):
    wl = configs.Workload(f"{cfg.name}_poison_b{B}", cfg, batch=B, seq_len=(8, 160), ragged=True, seed_batch=300 + B)
    bs = gen.make_batch(wl, extra_steps=1)
    weights = gen.make_weights(cfg, seed=tiny_seed()["seed"])
    pool = bits_to_torch(gen.bf16_bits(gen.make_kv_pool(cfg, bs.n_pages, seed=400 + B)))
    max_batch = B + 1 if B < 32 else B  # a row past the batch: never written by a step
    dec = make_decoder(cfg, bs, pool, int(bs.seq_lens.max()) + 1, mode, max_batch=max_batch)
    dec.load_weights({k: v.cuda() for k, v in weights.items()})
    tokens = bs.tokens.to(torch.int32).cuda()
    seq_lens = bs.seq_lens.to(torch.int32).cuda()
    bt = bs.block_tables.cuda()
    hint = int(bs.seq_lens.max())
    out = []
    for poison in (False, True, False):
        dec.set_debug_poison(poison)
        logits = torch.empty((B, cfg.vocab), dtype=torch.float32, device="cuda")
        nxt = torch.empty(B, dtype=torch.int32, device="cuda")
        if noalloc:
            dec.step(tokens, bt, seq_lens, hint, logits, nxt)  # builds the schedule (allocates)
            dec.sync()
            dec.step_noalloc(tokens, bt, seq_lens, hint, logits, nxt)
        else:
            dec.step(tokens, bt, seq_lens, hint, logits, nxt)
        dec.sync()
        h = dec.debug_read("h", (max_batch, cfg.hidden))
        out.append((logits.cpu().numpy(), nxt.cpu().numpy(), h))
    dec.close()
    return out


@pytest.mark.parametrize("cfg_name,B,mode,noalloc", [
    ("tiny_win", 1, 0, False), ("tiny_win", 4, 0, False), ("tiny_win", 32, 0, False),
    ("tiny_win", 4, 1, False), ("tiny_win", 1, 0, True), ("tiny_dense", 2, 0, False),
    ("layer1", 1, 0, False), ("layer1", 4, 0, False),
])
def test_poisoned_scratch_decodes_the_same_step(cfg_name, B, mode, noalloc):
    cfg = {"tiny_win": configs.TINY_WIN, "tiny_dense": configs.TINY_DENSE, "layer1": configs.LAYER1}[cfg_name]
    say(f"[poison] {cfg_name} B={B} mode={mode} noalloc={noalloc}")
    (l0, t0, h0), (l1, t1, h1), (l2, t2, h2) = _steps(cfg, B, mode, noalloc)
    assert np.all(np.isfinite(l0))
    assert np.array_equal(l0, l1) and np.array_equal(t0, t1)
    assert np.array_equal(l0, l2) and np.array_equal(t0, t2)
    if B < 32:
        # the residual stream's row past the batch: NaN only after the poisoned step
        assert np.all(np.isnan(h1[B])) and not np.any(np.isnan(h1[:B]))
        assert not np.any(np.isnan(h0[:B]))
