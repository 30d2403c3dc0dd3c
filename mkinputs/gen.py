"""Seeded synthetic inputs for one decode step: weights, KV cache, batch state.

This module only draws random numbers and lays them out; it holds none of the
decode step's arithmetic. Both the oracle (through numpy views) and the HIP
path (through device pointers) consume what it returns.

Recipe (random weights, as in the megakernel post's uniform-routing runs,
section "Decode throughput" of the Chinese version):
  * every matrix and the embedding: N(0, 0.02), rounded to bf16 (RNE);
  * RMSNorm gains: 1 + N(0, 0.02) in bf16, so a missing or mis-indexed gain shows;
  * synthetic context K and V: N(0, 1) in bf16;
  * tokens uniform over the vocabulary; ragged lengths uniform in a range;
  * page tables from a shuffled free-page pool.
Each tensor gets its own torch.Generator seeded from (base seed, tensor name),
so tensors are independent and each is reproducible on its own. Values depend
on the device they are drawn on (torch's CPU and GPU generators differ); a run
draws every input once and hands the same tensors to both sides.

Canonical layouts (row-major, [in x out]):
  emb [V, H]; gamma.{l} [H]; gamma_f [H]
  wqkv.{l} [H, QH*D + 2*KVH*D]   columns: q heads, then k heads, then v heads
  wo.{l} [QH*D, H]; wr.{l} [H, E]
  wg.{l}, wu.{l} [E, H, F]; wd.{l} [E, F, H]; wlm [H, V]
  dense models: gamma2.{l} [H] (the FFN's norm) in place of wr.{l}, E = 1,
  and wlm = emb transposed (tied)
KV pool (one page = page_size tokens, shared page ids across layers):
  pool [L, n_pages, 2, KVH, page_size*D] bf16, where plane 0 holds K with
  element (slot, d) at slot*D + d, and plane 1 holds V transposed, element
  (slot, d) at d*page_size + slot.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass
from typing import Dict, Optional

import numpy as np
import torch

from .configs import ModelConfig, Workload


def tensor_seed(base: int, name: str) -> int:
    h = hashlib.sha256(f"{base}:{name}".encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _normal_bf16(shape, seed: int, std: float, mean: float, device) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    x.mul_(std)
    if mean != 0.0:
        x.add_(mean)
    return x.to(torch.bfloat16)


def layer_kinds(m: ModelConfig) -> tuple:
    """The per-layer weight names of model m."""
    return DENSE_LAYER_KINDS if m.dense else LAYER_KINDS


def weight_shapes(m: ModelConfig) -> Dict[str, tuple]:
    H, E, F = m.hidden, m.n_experts, m.expert_ffn
    s = {"emb": (m.vocab, H), "gamma_f": (H,), "wlm": (H, m.vocab)}
    for l in range(m.n_layers):
        s[f"gamma.{l}"] = (H,)
        s[f"wqkv.{l}"] = (H, m.qkv_dim)
        s[f"wo.{l}"] = (m.q_dim, H)
        if m.dense:
            s[f"gamma2.{l}"] = (H,)
        else:
            s[f"wr.{l}"] = (H, E)
        s[f"wg.{l}"] = (E, H, F)
        s[f"wu.{l}"] = (E, H, F)
        s[f"wd.{l}"] = (E, F, H)
    return s


def weight_tensor(m: ModelConfig, name: str, seed: int = 1, device="cpu", std: float = 0.02,
                  expert: Optional[int] = None) -> torch.Tensor:
    """One canonical weight (or one expert's slice of an expert tensor), drawn
    exactly as make_weights draws it, so any piece can be regenerated alone."""
    shape = weight_shapes(m)[name]
    kind = name.split(".")[0]
    if m.dense and kind == "wlm":
        # tied: the LM head is the embedding matrix, [H, V]
        return weight_tensor(m, "emb", seed, device, std).t().contiguous()
    if kind.startswith("gamma"):
        return _normal_bf16(shape, tensor_seed(seed, name), std, 1.0, device)
    if kind in ("wg", "wu", "wd"):
        if expert is not None:
            return _normal_bf16(shape[1:], tensor_seed(seed, f"{name}.e{expert}"), std, 0.0, device)
        t = torch.empty(shape, dtype=torch.bfloat16, device=device)
        for e in range(shape[0]):
            t[e] = _normal_bf16(shape[1:], tensor_seed(seed, f"{name}.e{e}"), std, 0.0, device)
        return t
    return _normal_bf16(shape, tensor_seed(seed, name), std, 0.0, device)


LAYER_KINDS = ("gamma", "wqkv", "wo", "wr", "wg", "wu", "wd")
# a dense layer: attention norm, QKV, O, FFN norm, gate, up, down
DENSE_LAYER_KINDS = ("gamma", "wqkv", "wo", "gamma2", "wg", "wu", "wd")
GLOBAL_NAMES = ("emb", "gamma_f", "wlm")


def make_layer_weights(m: ModelConfig, layer: int, seed: int = 1, device="cpu") -> Dict[str, torch.Tensor]:
    return {f"{k}.{layer}": weight_tensor(m, f"{k}.{layer}", seed, device) for k in layer_kinds(m)}


def make_weights(m: ModelConfig, seed: int = 1, device="cpu", std: float = 0.02) -> Dict[str, torch.Tensor]:
    """All weights of model m as canonical bf16 tensors on `device`.

    Expert tensors are drawn one expert at a time (seed per expert slice) to
    bound the fp32 temporaries of the 48-layer model.
    """
    return {name: weight_tensor(m, name, seed, device, std) for name in weight_shapes(m)}


# ---------------------------------------------------------- FP8 weights
# Feed-forward weights handed over in FP8 (OCP E4M3) with one float32 scale
# per hidden unit and matrix: this prepares the inputs of a model stored that
# way (what a checkpoint converter would do); the decode step only ever reads
# the codes and scales.

E4M3_MAX = 448.0
FP8_KINDS = ("wg8", "wu8", "wd8", "sg", "su", "sd")


def quantize_ffn_fp8(wg: torch.Tensor, wu: torch.Tensor, wd: torch.Tensor):
    """FP8 codes and scales of FFN weights wg, wu [..., H, F] and wd [..., F, H]
    (bf16, on any device). Each hidden unit's gate column, up column and down
    row gets scale = max|w| / 448 (1 for an all-zero vector) and codes
    w / scale cast by torch to float8_e4m3fn (nearest, ties to even), clamped
    to +-448 first. Returns (cg, cu, cd) uint8 in the input layouts and
    (sg, su, sd) float32 [..., F]."""
    def q(w: torch.Tensor, axis: int):
        x = w.float()
        amax = x.abs().amax(dim=axis)
        scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
        y = (x / scale.unsqueeze(axis)).clamp_(-E4M3_MAX, E4M3_MAX)
        return y.to(torch.float8_e4m3fn).view(torch.uint8), scale
    cg, sg = q(wg, -2)
    cu, su = q(wu, -2)
    cd, sd = q(wd, -1)
    return cg, cu, cd, sg, su, sd


def add_fp8_ffn(m: ModelConfig, w: Dict[str, torch.Tensor], drop_bf16: bool = False) -> Dict[str, torch.Tensor]:
    """Add the FP8 form of every layer's FFN weights to w (names wg8.{l},
    wu8.{l}, wd8.{l}, sg.{l}, su.{l}, sd.{l}); with drop_bf16 the bf16 FFN
    tensors are removed. Returns w."""
    for l in range(m.n_layers):
        t = quantize_ffn_fp8(w[f"wg.{l}"], w[f"wu.{l}"], w[f"wd.{l}"])
        for k, v in zip(FP8_KINDS, t):
            w[f"{k}.{l}"] = v
        if drop_bf16:
            for k in ("wg", "wu", "wd"):
                del w[f"{k}.{l}"]
    return w


class LazyWeights:
    """Host bf16 bits of model weights, each drawn on `device` on first use
    (identical to make_weights on that device) and kept in host memory."""

    def __init__(self, m: ModelConfig, seed: int = 1, device="cuda", fp8: bool = False):
        self.m, self.seed, self.device, self.fp8 = m, seed, device, fp8
        if fp8:
            self.fp8_ffn = self._fp8_ffn
        self._c: Dict[tuple, np.ndarray] = {}
        self.overrides: Dict[tuple, np.ndarray] = {}

    def _fp8_ffn(self, layer: int, expert: int):
        """FP8 codes and scales of one FFN (quantize_ffn_fp8 of the drawn bf16
        weights, on `device`) as numpy arrays (bound as fp8_ffn when fp8)."""
        key = ("fp8", layer, expert)
        if key not in self._c:
            ws = [weight_tensor(self.m, f"{k}.{layer}", self.seed, self.device, expert=expert)
                  for k in ("wg", "wu", "wd")]
            self._c[key] = tuple(t.cpu().numpy() for t in quantize_ffn_fp8(*ws))
        return self._c[key]

    def __call__(self, name: str, layer: Optional[int] = None, expert: Optional[int] = None) -> np.ndarray:
        key = (name, layer, expert)
        if key in self.overrides:
            return self.overrides[key]
        if key not in self._c:
            full = name if layer is None else f"{name}.{layer}"
            self._c[key] = bf16_bits(weight_tensor(self.m, full, self.seed, self.device, expert=expert))
        return self._c[key]


@dataclass
class BatchState:
    tokens: torch.Tensor          # int32 [B]
    seq_lens: torch.Tensor        # int32 [B], counts the token being decoded
    block_tables: torch.Tensor    # int32 [B, max_pages_per_seq], -1 past the end
    n_pages: int                  # pages in the pool
    max_pages_per_seq: int


def make_batch(w: Workload, extra_steps: int = 0, device="cpu", spare_pages: int = 0,
               max_pages_per_seq: Optional[int] = None) -> BatchState:
    """Tokens, lengths and scattered page tables for workload w.

    Each sequence gets pages for seq_len + extra_steps positions, taken in
    order from a seeded permutation of the pool (the shuffled free list).
    """
    m = w.model
    P = m.page_size
    rng = np.random.Generator(np.random.Philox(tensor_seed(w.seed_batch, w.name)))
    B = w.batch
    lo, hi = w.seq_len
    if w.ragged:
        lens = rng.integers(lo, hi + 1, size=B)
    else:
        lens = np.full(B, lo)
    tokens = rng.integers(0, m.vocab, size=B)
    need = [-(-(int(n) + extra_steps) // P) for n in lens]
    mpps = max(need) if max_pages_per_seq is None else max_pages_per_seq
    assert mpps >= max(need)
    n_pages = sum(need) + spare_pages
    perm = rng.permutation(n_pages)
    bt = np.full((B, mpps), -1, dtype=np.int64)
    off = 0
    for b in range(B):
        bt[b, :need[b]] = perm[off:off + need[b]]
        off += need[b]
    return BatchState(
        tokens=torch.tensor(tokens, dtype=torch.int32, device=device),
        seq_lens=torch.tensor(lens, dtype=torch.int32, device=device),
        block_tables=torch.tensor(bt, dtype=torch.int32, device=device),
        n_pages=n_pages,
        max_pages_per_seq=mpps,
    )


def kv_pool_shape(m: ModelConfig, n_pages: int) -> tuple:
    return (m.n_layers, n_pages, 2, m.n_kv_heads, m.page_size * m.head_dim)


def make_kv_pool(m: ModelConfig, n_pages: int, seed: int = 2, device="cpu", fill: bool = True) -> torch.Tensor:
    """A KV pool filled with N(0, 1) bf16 (every slot of every page, per layer)."""
    shape = kv_pool_shape(m, n_pages)
    if not fill:
        return torch.zeros(shape, dtype=torch.bfloat16, device=device)
    pool = torch.empty(shape, dtype=torch.bfloat16, device=device)
    for l in range(m.n_layers):
        pool[l] = _normal_bf16(shape[1:], tensor_seed(seed, f"kv.{l}"), 1.0, 0.0, device)
    return pool


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """A bf16 tensor's raw bits as a numpy uint16 array (host copy)."""
    assert t.dtype == torch.bfloat16
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


class NumpyWeights:
    """Lazy host view of canonical weights as bf16 bit arrays.

    w(name) -> whole tensor; w(name, layer) -> per-layer tensor;
    w(name, layer, expert) -> one expert's slice. Fetches (and for device
    tensors, copies to the host) on first use.
    """

    def __init__(self, tensors: Dict[str, torch.Tensor], cache: bool = True):
        self.t = tensors
        self.cache = cache
        self._c: Dict[tuple, np.ndarray] = {}
        if "wg8.0" in tensors:
            self.fp8_ffn = self._fp8_ffn

    def _fp8_ffn(self, layer: int, expert: int):
        """One FFN's FP8 codes and scales (add_fp8_ffn's tensors) as numpy
        arrays: (cg, cu, cd, sg, su, sd); bound as fp8_ffn when present."""
        key = ("fp8", layer, expert)
        if key not in self._c:
            self._c[key] = tuple(self.t[f"{k}.{layer}"][expert].cpu().numpy() for k in FP8_KINDS)
        return self._c[key]

    def __call__(self, name: str, layer: Optional[int] = None, expert: Optional[int] = None) -> np.ndarray:
        key = (name, layer, expert)
        if key in self._c:
            return self._c[key]
        full = name if layer is None else f"{name}.{layer}"
        t = self.t[full]
        if expert is not None:
            t = t[expert]
        a = bf16_bits(t)
        if self.cache:
            self._c[key] = a
        return a

    def set(self, name: str, value_bits: np.ndarray, layer: Optional[int] = None):
        """Replace a whole tensor's bits (used when test inputs are adjusted)."""
        full = name if layer is None else f"{name}.{layer}"
        dev = self.t[full].device
        self.t[full] = torch.from_numpy(value_bits.view(np.int16).copy()).view(torch.bfloat16).to(dev)
        self._c = {k: v for k, v in self._c.items() if not (k[0] == name and k[1] == layer)}
