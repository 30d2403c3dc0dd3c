"""Shared test plumbing: build decoders and inputs, compare against the oracle.

Test infrastructure only. Inputs come from mkinputs (seeded), expected values
from oracle/; the HIP path is reached only through the C ABI binding.
"""
from __future__ import annotations

import json
import os
import sys
from dataclasses import dataclass

import numpy as np
import torch

from mkinputs import configs, gen

HERE = os.path.dirname(os.path.abspath(__file__))

LOGIT_MAX_ABS = 3e-2
LOGIT_REL_L2 = 1e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bits_to_torch(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def torch_to_bits(t: torch.Tensor) -> np.ndarray:
    return gen.bf16_bits(t)


def logits_close(gpu: np.ndarray, ref: np.ndarray):
    """(ok, max_abs, rel_l2) of one step's logits against the oracle."""
    d = gpu.astype(np.float64) - ref.astype(np.float64)
    mx = float(np.max(np.abs(d)))
    rl2 = float(np.linalg.norm(d) / max(np.linalg.norm(ref.astype(np.float64)), 1e-30))
    return (mx <= LOGIT_MAX_ABS and rl2 <= LOGIT_REL_L2), mx, rl2


def tiny_seed():
    return json.load(open(os.path.join(HERE, "golden", "tiny_seed.json")))


@dataclass
class TinyCase:
    wl: configs.Workload
    cfg: configs.ModelConfig
    weights: dict           # canonical CPU tensors
    W: gen.NumpyWeights
    bs: gen.BatchState
    ctx: np.ndarray          # [T, 1] context tokens


def tiny_case() -> TinyCase:
    rec = tiny_seed()
    wl = configs.WORKLOADS["tiny"]
    cfg = wl.model
    weights = gen.make_weights(cfg, seed=rec["seed"])
    bs = gen.make_batch(wl, extra_steps=wl.steps)
    rng = np.random.Generator(np.random.Philox(gen.tensor_seed(wl.seed_batch, "ctx")))
    ctx = rng.integers(0, cfg.vocab, size=(wl.seq_len[0] - 1, 1))
    return TinyCase(wl, cfg, weights, gen.NumpyWeights(weights), bs, ctx)


def make_decoder(cfg, bs: gen.BatchState, pool_gpu: torch.Tensor, max_seq_len: int, mode: int, max_batch=None):
    import moe_persistent_decode_amd as mk
    mc = mk.make_config(cfg, max_batch or bs.tokens.shape[0], max_seq_len, bs.n_pages, bs.max_pages_per_seq, mode)
    return mk.Decoder(mc, pool_gpu)


def router_repair_hook(cfg, gap: float = 2e-2, coords: int = 16, max_rounds: int = 400):
    """An oracle router_hook that widens every token's gap between its k-th and
    (k+1)-th router logit to at least `gap`, so the top-k set is decided by a
    margin well above two correct implementations' rounding differences.

    It moves the two experts' router columns apart by whole bf16 steps on the
    `coords` input coordinates of largest magnitude (the k-th expert's weights
    toward sign(x_i), the (k+1)-th's away from it), round after round, until
    every row clears the gap. Repaired matrices persist per layer (returned in
    the dict), so later steps start from them and the GPU can be given the
    same weights. Test-input construction only: the result is a valid weight
    matrix, not a change to the method.
    """
    from oracle import decode as od
    repaired = {}

    def bf16_step(bits, up):
        v = od.bf16_to_float(bits, np.float64)
        mag = np.abs(v)
        ulp = np.where(mag > 0, 2.0 ** (np.floor(np.log2(np.maximum(mag, 1e-38))) - 7), 2.0 ** -133)
        return od.float_to_bf16_rne((v + np.where(up, ulp, -ulp)).astype(np.float32))

    def hook(l, x, wr):
        wr = repaired.get(l, wr).copy()
        k = cfg.top_k
        changed = False
        for _ in range(max_rounds):
            r = x @ od.bf16_to_float(wr, x.dtype)
            done = True
            for b in range(r.shape[0]):
                order = np.argsort(-r[b], kind="stable")
                e_in, e_out = int(order[k - 1]), int(order[k])
                if r[b, e_in] - r[b, e_out] >= gap:
                    continue
                done = False
                top = np.argsort(-np.abs(x[b]))[:coords]
                pos = x[b, top] > 0
                wr[top, e_in] = bf16_step(wr[top, e_in], pos)
                wr[top, e_out] = bf16_step(wr[top, e_out], ~pos)
                changed = True
            if done:
                break
        else:
            raise AssertionError(f"router repair of layer {l} did not converge")
        if changed or l in repaired:
            repaired[l] = wr
        return wr

    return hook, repaired
