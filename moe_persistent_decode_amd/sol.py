"""Algorithmic bytes of one decode step and the HBM speed-of-light.

The megakernel post (section "What is a Megakernel?") measures decode against
a speed-of-light: the bytes a step must stream from HBM divided by the HBM
bandwidth (its example: 6.6 GB of active weights plus 0.5 GB of KV at 8K on a
3.35 TB/s part, about 470 tok/s). Here the bytes are counted exactly for one
step of the model actually decoded:

  per layer: QKV, O and router weights, the RMSNorm gain, the weights of each
  distinct expert the step routes to (gate, up and down; a dense layer: its
  second gain and its one FFN instead of router and experts), the KV read by each
  sequence (all positions for full-attention layers, at most the window for
  the others, the current token included), and the current token's K/V append;
  once: the LM head, the final gain, per sequence one embedding row and the
  float32 logits written.
Activations below a megabyte (hidden states, partial sums) are not counted.
"""
from __future__ import annotations

from typing import Sequence

MI355X_HBM_BYTES_PER_S = 8.0e12


def layer_weight_bytes(m) -> int:
    """Per layer: QKV and O projections and the norm gain; the router (MoE
    layers) or the second norm gain (dense layers). Expert or FFN weights are
    counted by step_bytes."""
    H = m.hidden
    if getattr(m, "dense", False):
        return 2 * (H * m.qkv_dim + m.q_dim * H + 2 * H)
    return 2 * (H * m.qkv_dim + m.q_dim * H + H * m.n_experts + H)


def expert_bytes(m, fp8: bool = False) -> int:
    """One expert's (or a dense layer's FFN) gate, up and down weights: bf16,
    or FP8 codes plus three float32 scales per hidden unit."""
    if fp8:
        return 3 * m.hidden * m.expert_ffn + 3 * 4 * m.expert_ffn
    return 2 * 3 * m.hidden * m.expert_ffn


def kv_bytes_per_token(m) -> int:
    return 2 * 2 * m.n_kv_heads * m.head_dim


def step_bytes(m, seq_lens: Sequence[int], n_active: Sequence[int], fp8: bool = False) -> int:
    """Algorithmic bytes of one step: seq_lens count the decoded token;
    n_active[l] = distinct experts routed to at layer l (1 for a dense
    layer's FFN); fp8: FP8 feed-forward weights."""
    B = len(seq_lens)
    kvt = kv_bytes_per_token(m)
    total = 0
    for l in range(m.n_layers):
        win = m.layer_window(l)
        kv_read = sum(min(int(s), win) if win else int(s) for s in seq_lens) * kvt
        total += layer_weight_bytes(m) + int(n_active[l]) * expert_bytes(m, fp8) + kv_read + B * kvt
    total += 2 * m.hidden * m.vocab + 2 * m.hidden + B * (2 * m.hidden + 4 * m.vocab)
    return total


def sol_tokens_per_s(bytes_per_step: float, batch: int, bw: float = MI355X_HBM_BYTES_PER_S) -> float:
    return batch * bw / bytes_per_step
