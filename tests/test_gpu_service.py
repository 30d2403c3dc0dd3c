"""The host decode service (mk_service_*) on the GPU, tiny model.

Megakernel post, Chinese version, engine section: a native thread decodes the
batch step after step and streams tokens, while the control plane pauses it
(park), changes the batch (admit, evict, prefill into KV pages) and resumes
it. Three requests with synthetic contexts written into pages the service
hands out: two decode first; the service is paused mid-stream, a third is
admitted and the second evicted; decoding resumes. Every streamed token
equals the oracle's greedy decode of that request on its own (contexts in
contiguous pages: paged equals contiguous); the evicted request's tokens are
a prefix of its oracle run; every page returns to the free list.

The weights are repaired before the run (router and LM-head margin repairs
through the oracle's hooks, repeated over all requests until no decision of
any request moves), so every routing and greedy decision has a margin of at
least 2e-2 and the comparison is exact.
"""
import time

import numpy as np
import pytest
import torch

import moe_persistent_decode_amd as mk
from mkinputs import configs, gen
from oracle import decode as od
from oracle import trajectory as tj
from tests.harness import bits_to_torch, lm_repair_hook, router_repair_hook, say, tiny_seed

pytestmark = pytest.mark.gpu

P = 16
REQS = [  # (id, context length, first token, tokens to decode)
    (11, 40, 101, 12),
    (22, 70, 202, 12),
    (33, 25, 303, 8),
]


def _context(cfg, ctx_len, seed):
    """Synthetic context K/V for positions < ctx_len: [L][pages][2][KVH][P*D] bf16 bits."""
    n = -(-ctx_len // P)
    return gen.bf16_bits(gen.make_kv_pool(cfg, n, seed=seed))


def _oracle(cfg, W, ctx, first, ctx_len, steps, hooks):
    n_pages = -(-(ctx_len + steps) // P)
    pool = np.zeros(gen.kv_pool_shape(cfg, n_pages), dtype=np.uint16)
    pool[:, :ctx.shape[1]] = ctx
    bt = np.arange(n_pages)[None, :]
    return tj.greedy_decode(cfg, W, pool, bt, np.array([first]), np.array([ctx_len + 1]), steps, **hooks)


def test_decode_service_streams_the_oracles_tokens():
    cfg = configs.TINY
    weights = gen.make_weights(cfg, seed=tiny_seed()["seed"])
    ctxs = {rid: _context(cfg, n, seed=500 + rid) for rid, n, _, _ in REQS}
    # repair the weights until every request's decisions clear the margins
    rh, rrep = router_repair_hook(cfg)
    lh, lst = lm_repair_hook()
    for _ in range(10):
        before = ({l: w.copy() for l, w in rrep.items()}, None if lst["wlm"] is None else lst["wlm"].copy())
        W = gen.NumpyWeights(weights)
        for rid, n, first, steps in REQS:
            _oracle(cfg, W, ctxs[rid], first, n, steps, dict(router_hook=rh, lm_hook=lh))
        same = before[0].keys() == rrep.keys() and all(np.array_equal(before[0][l], rrep[l]) for l in rrep) and \
            (before[1] is None) == (lst["wlm"] is None) and (before[1] is None or np.array_equal(before[1], lst["wlm"]))
        if same:
            break
    else:
        raise AssertionError("repairs did not settle")
    for l, wr in rrep.items():
        weights[f"wr.{l}"] = torch.from_numpy(wr.view(np.int16).copy()).view(torch.bfloat16)
    if lst["wlm"] is not None:
        weights["wlm"] = torch.from_numpy(lst["wlm"].view(np.int16).copy()).view(torch.bfloat16)
    W = gen.NumpyWeights(weights)
    ref = {}
    for rid, n, first, steps in REQS:
        run = _oracle(cfg, W, ctxs[rid], first, n, steps, {})
        assert run.min_greedy_gap() >= 2e-2 * (1 - 1e-4) and run.min_router_gap(cfg.top_k) >= 2e-2 * (1 - 1e-4)
        ref[rid] = [int(g[0]) for g in run.greedy]

    n_pages = 48
    mpps = 8
    pool = torch.zeros(gen.kv_pool_shape(cfg, n_pages), dtype=torch.bfloat16, device="cuda")
    dec = mk.Decoder(mk.make_config(cfg, 4, mpps * P, n_pages, mpps, 0), pool)
    svc = None
    try:
        dec.load_weights({k: v.cuda() for k, v in weights.items()})
        svc = mk.DecodeService(dec, max_batch=4, page0=0, n_pages=n_pages)
        assert svc.stats().parked == 1

        def admit(rid, n, first, steps):
            ctx = ctxs[rid]
            pages = svc.alloc_pages(ctx.shape[1])
            pool[:, pages] = bits_to_torch(ctx)  # the "prefill": context K/V into the service's pages
            torch.cuda.synchronize()
            svc.admit(rid, first, n, pages, steps)

        admit(*REQS[0])
        admit(*REQS[1])
        svc.resume()
        t0 = time.time()
        while len(svc.snapshot()[0].get(22, [])) < 4:
            assert time.time() - t0 < 60, "no tokens streamed"
            time.sleep(0.002)
        svc.pause()
        toks, _ = svc.snapshot()
        n22 = len(toks[22])
        say(f"[service] paused after {n22} tokens of request 22; admit 33, evict 22")
        svc.evict(22)
        admit(*REQS[2])
        svc.resume()
        t0 = time.time()
        while True:
            toks, status = svc.snapshot()
            if status.get(11) == 1 and status.get(33) == 1:
                break
            assert -1 not in status.values(), svc.stats().status
            assert time.time() - t0 < 60, "requests did not finish"
            time.sleep(0.002)
        st = svc.stats()
        say(f"[service] steps {st.steps}, tokens {st.tokens}; 11: {toks[11]} 33: {toks[33]}")
        assert toks[11] == ref[11] and toks[33] == ref[33]
        assert toks[22] == ref[22][:len(toks[22])] and len(toks[22]) == n22 and 22 not in status
        # idle again, every page back on the free list
        t0 = time.time()
        while not svc.stats().parked:
            assert time.time() - t0 < 10
            time.sleep(0.001)
        st = svc.stats()
        assert st.active == 0 and st.free_pages == n_pages and st.status == 0
    finally:
        if svc is not None:
            svc.close()
        dec.close()
