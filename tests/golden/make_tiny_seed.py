"""Pick the weight seed of the tiny decode case and record its margins.

Calls only `oracle` and `mkinputs`. The tiny case is a 2-layer model decoded
greedily for 16 steps after a 128-token context of uniform random tokens.
The chosen seed is the first one for which every decision the GPU must
reproduce bit-exactly has a margin in the oracle of at least:
  * 1e-2 for the routing (k-th vs (k+1)-th router logit) and greedy
    (top-1 vs top-2 logit) decisions of the 16 decode steps and for the
    greedy token that ends the context;
  * 2e-4 for the routing decisions made while the context is built token by
    token (exercised only when the GPU rebuilds the context itself; the two
    sides' router logits differ by accumulation order, about 1e-6).
Run: python tests/golden/make_tiny_seed.py  (writes tests/golden/tiny_seed.json)
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from mkinputs import configs, gen  # noqa: E402
from oracle import trajectory as tj  # noqa: E402

DECODE_MARGIN = 1e-2
CONTEXT_MARGIN = 2e-4


def tiny_case(seed):
    wl = configs.WORKLOADS["tiny"]
    cfg = wl.model
    W = gen.NumpyWeights(gen.make_weights(cfg, seed=seed))
    bs = gen.make_batch(wl, extra_steps=wl.steps)
    rng = np.random.Generator(np.random.Philox(gen.tensor_seed(wl.seed_batch, "ctx")))
    ctx = rng.integers(0, cfg.vocab, size=(wl.seq_len[0] - 1, 1))
    return wl, cfg, W, bs, ctx


def evaluate(seed):
    wl, cfg, W, bs, ctx = tiny_case(seed)
    bt = bs.block_tables.numpy()
    pool = np.zeros(gen.kv_pool_shape(cfg, bs.n_pages), np.uint16)
    c = tj.teacher_forced(cfg, W, pool, bt, ctx, np.array([1]))
    g0 = c.greedy[-1]
    d = tj.greedy_decode(cfg, W, pool, bt, g0, np.array([wl.seq_len[0]]), wl.steps)
    return {
        "seed": seed,
        "context_router_gap": c.min_router_gap(cfg.top_k),
        "context_last_greedy_gap": float(tj.greedy_gap(c.logits[-1]).min()),
        "decode_router_gap": d.min_router_gap(cfg.top_k),
        "decode_greedy_gap": d.min_greedy_gap(),
        "first_token": int(g0[0]),
        "greedy_tokens": [int(t[0]) for t in d.greedy],
    }


def accepted(m):
    return (m["decode_router_gap"] >= DECODE_MARGIN and m["decode_greedy_gap"] >= DECODE_MARGIN
            and m["context_last_greedy_gap"] >= DECODE_MARGIN
            and m["context_router_gap"] >= CONTEXT_MARGIN
            and len(set(m["greedy_tokens"])) >= 2)


if __name__ == "__main__":
    for s in range(1, 200):
        m = evaluate(s)
        if accepted(m):
            m["thresholds"] = {"decode": DECODE_MARGIN, "context": CONTEXT_MARGIN}
            with open(os.path.join(HERE, "tiny_seed.json"), "w") as fh:
                json.dump(m, fh, indent=1)
            print(m)
            break
