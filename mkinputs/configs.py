"""Model shapes and workloads of the synthetic decode inputs.

These are plain data: the shapes of a parallel-transformer MoE decoder and the
batch/context mixes it is decoded at. Both the oracle and the HIP path read
them; neither's arithmetic lives here.

Shapes of the full-size model (hidden 2048, 32 query heads over 4 key/value
groups of head_dim 128, 128 experts with top-8 routing, expert width 768, vocab
131072, 48 layers of which 12 use full attention and 36 a 4096-token sliding
window) are the ones the Cohere North Mini Code megakernel post implies
(section "What is a Megakernel?": 30B total / 3.3B active, 0.5 GB of KV at 8K;
section "Tasks": 128 experts, top-8; section "Drop false dependencies": 4
key/value groups). Layer l uses full attention iff l % 4 == 3; RoPE theta 1e4
and RMSNorm eps 1e-6 are readings (the pages give neither).
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Tuple


@dataclass(frozen=True)
class ModelConfig:
    name: str
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_experts: int
    top_k: int
    expert_ffn: int
    vocab: int
    n_layers: int
    rope_theta: float = 1e4
    eps: float = 1e-6
    page_size: int = 16
    window: int = 0          # 0: every layer attends to the whole context
    full_every: int = 1      # with window > 0, layer l is full iff l % full_every == full_every - 1
    # dense: a sequential layer (attention, then a second RMSNorm and one
    # SwiGLU FFN of width expert_ffn; n_experts = top_k = 1, no router) and an
    # LM head tied to the embedding
    dense: bool = False

    @property
    def q_dim(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def qkv_dim(self) -> int:
        return self.q_dim + 2 * self.kv_dim

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    def is_full(self, layer: int) -> bool:
        return self.window == 0 or (layer % self.full_every) == self.full_every - 1

    def layer_window(self, layer: int) -> int:
        """0 for a full-attention layer, else the window length in tokens."""
        return 0 if self.is_full(layer) else self.window

    def param_counts(self) -> Tuple[int, int]:
        """(total, active per token) parameter counts, untied embedding and LM
        head (a dense model's tied matrix counted once)."""
        H, E, F = self.hidden, self.n_experts, self.expert_ffn
        attn = H * self.qkv_dim + self.q_dim * H
        if self.dense:
            total = self.n_layers * (attn + 3 * H * F + 2 * H) + self.vocab * H + H
            return total, total
        router = H * E
        expert = 3 * H * F
        norms = H
        per_layer_total = attn + router + E * expert + norms
        per_layer_active = attn + router + self.top_k * expert + norms
        emb = self.vocab * H
        lm = H * self.vocab
        total = self.n_layers * per_layer_total + emb + lm + H
        active = self.n_layers * per_layer_active + emb + lm + H
        return total, active


TINY = ModelConfig(name="tiny", hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                   n_experts=8, top_k=2, expert_ffn=128, vocab=1024, n_layers=2)

# the tiny shapes with a sliding window: layer 0 attends to the 48 most recent
# positions (three pages, not page-aligned in general), layer 1 to all
TINY_WIN = ModelConfig(name="tiny_win", hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                       n_experts=8, top_k=2, expert_ffn=128, vocab=1024, n_layers=2,
                       window=48, full_every=2)

LAYER1 = ModelConfig(name="layer1", hidden=2048, n_q_heads=32, n_kv_heads=4, head_dim=128,
                     n_experts=128, top_k=8, expert_ffn=768, vocab=131072, n_layers=1)

FULL48 = ModelConfig(name="full48", hidden=2048, n_q_heads=32, n_kv_heads=4, head_dim=128,
                     n_experts=128, top_k=8, expert_ffn=768, vocab=131072, n_layers=48,
                     window=4096, full_every=4)

# A dense decoder shaped like Llama-3.2-1B (the model of the Hazy Research
# megakernel the megakernel post starts from, section "Where we started", and
# of the tiny-vllm walkthrough: hidden 2048, 16 layers, 2048-wide q and
# 512-wide k/v projections of head_dim 64, vocab 128256, RoPE theta 500000,
# logits from the embedding matrix). The FFN width 8192 and eps 1e-5 are
# readings (the model's published configuration; the pages give neither).
# Random weights: the shapes are what the decode step's cost depends on.
LLAMA1B = ModelConfig(name="llama1b", hidden=2048, n_q_heads=32, n_kv_heads=8, head_dim=64,
                      n_experts=1, top_k=1, expert_ffn=8192, vocab=128256, n_layers=16,
                      rope_theta=500000.0, eps=1e-5, dense=True)

TINY_DENSE = ModelConfig(name="tiny_dense", hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                         n_experts=1, top_k=1, expert_ffn=512, vocab=1024, n_layers=2,
                         rope_theta=500000.0, eps=1e-5, dense=True)


@dataclass(frozen=True)
class Workload:
    """A batch of sequences decoded together.

    seq_len: length of each sequence at the first decode step, counting the
    token being decoded (its position is seq_len - 1); a (lo, hi) range drawn
    uniformly per sequence when ragged is True, else (n, n).
    """
    name: str
    model: ModelConfig
    batch: int
    seq_len: Tuple[int, int]
    ragged: bool = False
    steps: int = 1
    seed_weights: int = 1
    seed_kv: int = 2
    seed_batch: int = 3


WORKLOADS = {
    # 2-layer tiny model: 128-token context, 16 greedy steps (correctness case)
    "tiny": Workload("tiny", TINY, batch=1, seq_len=(129, 129), steps=16),
    # one full-size full-attention layer, 8K context, batch 1
    "layer1_b1_8k": Workload("layer1_b1_8k", LAYER1, batch=1, seq_len=(8192, 8192), steps=16),
    # the 48-layer model at batch 1, 8K context
    "full48_b1_8k": Workload("full48_b1_8k", FULL48, batch=1, seq_len=(8192, 8192), steps=256),
    # batches 2 and 4 at 8K (the scheduler ablation's batch sizes)
    "full48_b2_8k": Workload("full48_b2_8k", FULL48, batch=2, seq_len=(8192, 8192), steps=64),
    "full48_b4_8k": Workload("full48_b4_8k", FULL48, batch=4, seq_len=(8192, 8192), steps=64),
    # batch 32, ragged contexts U{512..16384}
    "full48_b32_ragged": Workload("full48_b32_ragged", FULL48, batch=32, seq_len=(512, 16384),
                                  ragged=True, steps=16),
    # the one-layer model at the long-context shapes (parity cases)
    "layer1_b1_256k": Workload("layer1_b1_256k", LAYER1, batch=1, seq_len=(262144, 262144), steps=4),
    "layer1_b4_64k": Workload("layer1_b4_64k", LAYER1, batch=4, seq_len=(65536, 65536), steps=4),
    "layer1_b32_ragged": Workload("layer1_b32_ragged", LAYER1, batch=32, seq_len=(512, 16384),
                                  ragged=True, steps=4),
    # long context
    "full48_b1_256k": Workload("full48_b1_256k", FULL48, batch=1, seq_len=(262144, 262144), steps=64),
    "full48_b4_64k": Workload("full48_b4_64k", FULL48, batch=4, seq_len=(65536, 65536), steps=64),
    # the dense Llama-3.2-1B-shaped decoder at batch 1 and 4, 8K context
    "llama1b_b1_8k": Workload("llama1b_b1_8k", LLAMA1B, batch=1, seq_len=(8192, 8192), steps=64),
    "llama1b_b4_ragged": Workload("llama1b_b4_ragged", LLAMA1B, batch=4, seq_len=(512, 16384),
                                  ragged=True, steps=16),
    "tiny_dense": Workload("tiny_dense", TINY_DENSE, batch=1, seq_len=(129, 129), steps=16),
}


def small_variant(model: ModelConfig, **kw) -> ModelConfig:
    """A copy of a model with some fields replaced (used for reduced test shapes)."""
    return replace(model, **kw)
