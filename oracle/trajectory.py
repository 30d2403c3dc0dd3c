"""Multi-step decoding with the oracle, and the decision margins of a run.

TEST INFRASTRUCTURE ONLY (see the package docstring).

A decode step is a pure function of (weights, KV cache, page tables, tokens,
lengths) whose only lasting effect is the K/V append; stepping again with
lengths + 1 continues decoding (megakernel post, Chinese version, section on
the engine around the kernel: the C++ loop updates KV positions, launches,
samples greedily and repeats). Routing decisions and greedy tokens are integer
results decided by floating point, so the parity tests need every such
decision to have a margin well above the rounding differences between two
correct implementations; these helpers measure those margins.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List

import numpy as np

from .decode import decode_step, greedy


def router_gap(r: np.ndarray, k: int) -> np.ndarray:
    """Gap between the k-th and (k+1)-th largest router logits, per row."""
    s = -np.sort(-np.asarray(r, dtype=np.float64), axis=-1)
    if s.shape[-1] <= k:
        return np.full(s.shape[:-1], np.inf)
    return s[..., k - 1] - s[..., k]


def greedy_gap(logits: np.ndarray) -> np.ndarray:
    """Gap between the largest and second largest logit, per row."""
    s = -np.sort(-np.asarray(logits, dtype=np.float64), axis=-1)
    return s[..., 0] - s[..., 1]


@dataclass
class Run:
    tokens_in: List[np.ndarray] = field(default_factory=list)     # per step [B]
    seq_lens: List[np.ndarray] = field(default_factory=list)      # per step [B]
    logits: List[np.ndarray] = field(default_factory=list)        # per step [B, V]
    greedy: List[np.ndarray] = field(default_factory=list)        # per step [B]
    traces: list = field(default_factory=list)

    def min_router_gap(self, k: int) -> float:
        g = [router_gap(r, k).min() for tr in self.traces for r in tr.router_logits]
        return float(min(g)) if g else float("inf")

    def min_greedy_gap(self) -> float:
        return float(min(greedy_gap(lg).min() for lg in self.logits))


def teacher_forced(cfg, W, pool, block_tables, tokens_per_step, seq_len0, dtype=np.float32, **hooks) -> Run:
    """Feed given tokens step by step (tokens_per_step [T, B]) from lengths seq_len0.
    hooks: router_hook / lm_hook, passed to every decode_step."""
    run = Run()
    lens = np.asarray(seq_len0).copy()
    for toks in tokens_per_step:
        toks = np.asarray(toks)
        lg, tr = decode_step(cfg, W, pool, block_tables, toks, lens, dtype=dtype, **hooks)
        run.tokens_in.append(toks); run.seq_lens.append(lens.copy())
        run.logits.append(lg); run.greedy.append(greedy(lg)); run.traces.append(tr)
        lens = lens + 1
    return run


def greedy_decode(cfg, W, pool, block_tables, first_tokens, seq_len0, steps, dtype=np.float32, **hooks) -> Run:
    """Decode `steps` greedy steps: each step's argmax is the next step's token.
    hooks: router_hook / lm_hook, passed to every decode_step."""
    run = Run()
    toks = np.asarray(first_tokens).copy()
    lens = np.asarray(seq_len0).copy()
    for _ in range(steps):
        lg, tr = decode_step(cfg, W, pool, block_tables, toks, lens, dtype=dtype, **hooks)
        run.tokens_in.append(toks.copy()); run.seq_lens.append(lens.copy())
        nxt = greedy(lg)
        run.logits.append(lg); run.greedy.append(nxt); run.traces.append(tr)
        toks = nxt
        lens = lens + 1
    return run
