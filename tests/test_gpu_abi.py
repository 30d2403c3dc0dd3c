"""GPU tests of the boundary's own behaviour, through the C ABI.

- A library-owned KV pool (mk_create with no pool): the caller writes the
  context into each layer's part through the address mk_kv_cache gives, and
  the step matches the oracle.
- Forced wait timeouts: with a one-microsecond limit on every dependency
  wait, a step at batch 32 gives up (each wait is bounded, every workgroup
  drains its list and the kernel exits); mk_sync_status reports
  MK_ERR_DEVICE_TIMEOUT, and the same step run again with the default limit
  matches the oracle.
- A row whose logits are all NaN has no greedy token: the step reports
  MK_ERR_DEVICE_FAULT instead of publishing one, and with a valid LM head the
  next step matches the oracle.
"""
import ctypes

import numpy as np
import pytest
import torch

import moe_persistent_decode_amd as mk
from mkinputs import configs, gen
from oracle import decode as od
from tests.harness import bits_to_torch, logits_close, make_decoder, say, tiny_seed

pytestmark = pytest.mark.gpu


def _hip_copy_d2d(dst: int, src: int, nbytes: int):
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    assert hip.hipMemcpy(dst, src, nbytes, 3) == 0  # hipMemcpyDeviceToDevice


def _tiny_batch(B, seed, lo=20, hi=150):
    cfg = configs.TINY
    wl = configs.Workload(f"tiny_abi_b{B}", cfg, batch=B, seq_len=(lo, hi), ragged=True, seed_batch=seed)
    bs = gen.make_batch(wl, extra_steps=2)
    weights = gen.make_weights(cfg, seed=tiny_seed()["seed"])
    pool = gen.bf16_bits(gen.make_kv_pool(cfg, bs.n_pages, seed=seed + 100))
    return cfg, bs, weights, pool


def _step(dec, bs, B, logits, nxt):
    dec.step(bs.tokens.cuda(), bs.block_tables.cuda(), bs.seq_lens.cuda(), int(bs.seq_lens.max()), logits, nxt)


def _compare(cfg, bs, weights, pool, lg, tok):
    ref, _ = od.decode_step(cfg, gen.NumpyWeights(weights), pool.copy(), bs.block_tables.numpy(),
                            bs.tokens.numpy(), bs.seq_lens.numpy())
    gaps = np.sort(ref, axis=-1)
    for b in range(lg.shape[0]):
        ok, mx, rl2 = logits_close(lg[b], ref[b])
        assert ok, (b, mx, rl2)
        if gaps[b, -1] - gaps[b, -2] >= 1e-2:
            assert int(tok[b]) == int(np.argmax(ref[b])), b
    return ref


def test_library_owned_kv_pool():
    cfg, bs, weights, pool = _tiny_batch(4, seed=81)
    mc = mk.make_config(cfg, 4, int(bs.seq_lens.max()) + 2, bs.n_pages, bs.max_pages_per_seq, 0)
    dec = mk.Decoder(mc, None)
    try:
        src = bits_to_torch(pool)
        per = src[0].numel() * 2
        base0, n0 = dec.kv_cache(0)
        for l in range(cfg.n_layers):
            base, n = dec.kv_cache(l)
            assert n == per and base == base0 + l * per
            _hip_copy_d2d(base, src[l].data_ptr(), n)
        torch.cuda.synchronize()
        dec.load_weights({k: v.cuda() for k, v in weights.items()})
        logits = torch.empty((4, cfg.vocab), dtype=torch.float32, device="cuda")
        nxt = torch.empty(4, dtype=torch.int32, device="cuda")
        _step(dec, bs, 4, logits, nxt)
        dec.sync()
        _compare(cfg, bs, weights, pool, logits.cpu().numpy(), nxt.cpu().numpy())
        say("[abi] library-owned pool: step matches the oracle")
    finally:
        dec.close()


def test_forced_wait_timeouts_drain_and_the_next_step_is_clean():
    B = 32
    cfg, bs, weights, pool = _tiny_batch(B, seed=83)
    pool_gpu = bits_to_torch(pool)
    dec = make_decoder(cfg, bs, pool_gpu, int(bs.seq_lens.max()) + 2, 0, max_batch=B)
    try:
        dec.load_weights({k: v.cuda() for k, v in weights.items()})
        logits = torch.empty((B, cfg.vocab), dtype=torch.float32, device="cuda")
        nxt = torch.empty(B, dtype=torch.int32, device="cuda")
        dec.set_wait_limit(1)
        _step(dec, bs, B, logits, nxt)
        with pytest.raises(mk.MkError) as e:
            dec.sync()
        assert e.value.status == 5, str(e.value)  # MK_ERR_DEVICE_TIMEOUT
        say(f"[abi] forced timeouts: {e.value}")
        dec.set_wait_limit(0)
        _step(dec, bs, B, logits, nxt)  # the same step again (it rewrites the same K/V slots)
        dec.sync()
        _compare(cfg, bs, weights, pool, logits.cpu().numpy(), nxt.cpu().numpy())
        say("[abi] the step after the timeouts matches the oracle")
    finally:
        dec.close()


def test_all_nan_logits_raise_a_fault():
    cfg, bs, weights, pool = _tiny_batch(2, seed=85)
    pool_gpu = bits_to_torch(pool)
    dec = make_decoder(cfg, bs, pool_gpu, int(bs.seq_lens.max()) + 2, 0, max_batch=2)
    try:
        w = {k: v.cuda() for k, v in weights.items()}
        dec.load_weights(w)
        nan_lm = torch.full_like(w["wlm"], float("nan"))
        dec.load_globals(w["emb"], w["gamma_f"], nan_lm)
        logits = torch.empty((2, cfg.vocab), dtype=torch.float32, device="cuda")
        nxt = torch.full((2,), -7, dtype=torch.int32, device="cuda")
        _step(dec, bs, 2, logits, nxt)
        with pytest.raises(mk.MkError) as e:
            dec.sync()
        assert e.value.status == 6, str(e.value)  # MK_ERR_DEVICE_FAULT
        assert nxt.cpu().tolist() == [-7, -7]     # no token was published
        say(f"[abi] all-NaN logits: {e.value}")
        dec.load_globals(w["emb"], w["gamma_f"], w["wlm"])
        _step(dec, bs, 2, logits, nxt)
        dec.sync()
        _compare(cfg, bs, weights, pool, logits.cpu().numpy(), nxt.cpu().numpy())
    finally:
        dec.close()


def test_stream_read_runs_and_writes_nothing():
    """The streaming-read diagnostic reads a buffer (a ragged length of
    16-byte words, so both of its loops run) and leaves it unchanged."""
    import moe_persistent_decode_amd as mk
    say("[abi] stream_read over 64 MiB + 48 bytes")
    buf = torch.arange((64 << 20) // 4 + 12, dtype=torch.int32, device="cuda")
    ref = buf.clone()
    mk.stream_read(buf)
    torch.cuda.synchronize()
    assert torch.equal(buf, ref)


def test_cross_xcd_message_passing_sees_no_stale_read():
    """The hand-off protocol of every task (device-coherent stores, a drain, a
    relaxed device-scope counter increment; polls and device-coherent reads on
    the other side) between 128 workgroup pairs on different XCDs, 2000
    messages each: no stale word, no wait that gave up. The tagged-word
    hand-off (value and tag in one 8-byte store, no drain or counter; the
    reader polls the words): every value read belongs to its tag. The same run with
    plain accesses for the message is reported for contrast (not asserted:
    whether a stale line is seen there depends on timing)."""
    import moe_persistent_decode_amd as mk
    say("[abi] cross-XCD message passing: 128 pairs x 2000 rounds")
    stale, timeouts = mk.litmus_message_passing(128, 2000, coherent=True)
    say(f"  device-coherent: stale {stale}, timeouts {timeouts}")
    assert stale == 0 and timeouts == 0
    stale_t, timeouts_t = mk.litmus_message_passing(128, 2000, coherent="tagged")
    say(f"  tagged words: torn {stale_t}, timeouts {timeouts_t}")
    assert stale_t == 0 and timeouts_t == 0
    stale_p, timeouts_p = mk.litmus_message_passing(128, 2000, coherent=False)
    say(f"  plain accesses: stale {stale_p}, timeouts {timeouts_p}")
