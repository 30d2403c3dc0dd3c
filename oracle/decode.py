"""One decode step, written out as its plain definition (numpy, CPU).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources. "Megakernel post" is Cohere's post on the North Mini Code decode
megakernel (English page and its Chinese version); "tiny-vllm walkthrough" is
the code-series article "5. The decode path that produces one token - why
separate kernels were made".

The model (megakernel post, section "Reduce wave quantization" with its Image
4, and section "Tasks"): a parallel transformer layer. Attention and the MoE
feed-forward both read the same RMS-normalised input, and their outputs are
added back to the residual stream together:

    x  = RMSNorm(h; gamma_l)
    h <- h + Attention(x) + MoE(x)

Attention: QKV projection with RoPE applied to q and k, grouped-query
attention over a paged bf16 KV cache (4 key/value groups, section "Drop false
dependencies"), O projection. MoE: a router scores the experts, the top-k are
kept, and each token's k expert outputs are summed weighted by its router
scores (section "Tasks", MoE routing and MoE GEMMs). After the last layer a
final RMSNorm and the LM head give the logits; decoding is greedy.

The second model is dense and sequential, shaped like Llama-3.2-1B (the
model of the Hazy Research megakernel the post starts from, section "Where
we started", and of the tiny-vllm walkthrough, section "The remaining layers
and logits"):

    h <- h + Attention(RMSNorm(h; gamma_l))
    h <- h + FFN(RMSNorm(h; gamma2_l))

with one SwiGLU FFN per layer (section "Tasks": FFN_UPGATE_ACT fuses the
SiLU-and-multiply, FFN_DOWN) and logits from the embedding matrix (tiny-vllm:
the logits come from embed_tokens).

Readings where the pages are silent (all fixed here, listed in the design doc):
  R1  seq_lens counts the token being decoded; its position is seq_len - 1,
      and its K/V are written into the cache before attention reads it
      (tiny-vllm walkthrough, "The decode loop: where it starts").
  R2  Page p of a sequence holds positions [16p, 16p+16); position j lives in
      page block_table[j // 16], slot j % 16 (tiny-vllm walkthrough,
      "Gathering K/V into a batched buffer and scattering into blocks").
  R3  RMSNorm: h / sqrt(mean(h^2) + eps) * gamma, eps = 1e-6; L+1 gains.
  R4  RoPE on interleaved pairs (2i, 2i+1), frequency theta^(-2i/D), the
      angle position * frequency formed in float64 (tiny-vllm walkthrough,
      "RoPE: one current position, recomputed on every call", pairs 2i, 2i+1).
  R5  Query head h reads key/value group h // (QH / KVH).
  R6  Full-attention layers read positions [0, p]; window layers read the W
      most recent positions including the current one, [max(0, p-W+1), p].
  R7  Scores scaled by 1/sqrt(D); no biases, no QK-norm, no softcap.
  R8  Top-k by router logit, ties to the lower expert index; weights are the
      softmax of the k kept logits (a softmax renormalised over the top-k).
  R9  Expert FFN: (silu(x Wg) * (x Wu)) Wd, silu(z) = z / (1 + exp(-z)).
  R10 K and V enter the cache rounded to bf16 (round to nearest even);
      activations stay in the working precision; logits are float32.
  R11 Greedy token: argmax of the logits, the lowest index on ties
      (tiny-vllm walkthrough, "The remaining layers and logits": the scan
      replaces the running best only on a strictly greater value).
  R19, R20 (FP8 feed-forward weights: the format and the scales): in the
      fp8 section below.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Callable, List, Optional

import numpy as np


# ---------------------------------------------------------------- bf16 ------

def bf16_to_float(bits: np.ndarray, dtype=np.float32) -> np.ndarray:
    """bf16 bit patterns -> float (exact: a bf16 is the top half of a float32)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(dtype, copy=False)


def float_to_bf16_rne(x: np.ndarray) -> np.ndarray:
    """float -> bf16 bits, round to nearest, ties to even (R10). NaN stays NaN."""
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        r = np.where(nan, np.uint16(0x7FC0), r)
    return r


# ---------------------------------------------------------------- fp8 ------
# FP8 weights are the post's next step (Chinese version, section "下一步":
# FP8 and FP4 quantization on the roadmap; section on the other schedulers:
# narrower types such as FP8). The pages fix neither the format nor the
# scaling; the readings taken here (listed in the design doc):
#   R19 The format is the OCP 8-bit floating point E4M3 ("FN": one sign bit,
#       a 4-bit exponent of bias 7, a 3-bit mantissa; exponent field 0 holds
#       the subnormals m * 2^-9; S.1111.111 is NaN; no infinities; largest
#       finite magnitude 448).
#   R20 Only the feed-forward weights are FP8 (each expert's gate, up and
#       down matrices, or a dense layer's FFN): they are the bytes a decode
#       step streams most of. Each hidden unit f of an FFN has three float32
#       scales: its gate column, its up column and its down row are
#       code value * scale (Wg[k, f] = e4m3(Cg[k, f]) * sg[f],
#       Wu[k, f] = e4m3(Cu[k, f]) * su[f], Wd[f, n] = e4m3(Cd[f, n]) * sd[f]).
#       The rest of the step is as for bf16 weights.

def _e4m3_fields(c: np.ndarray) -> np.ndarray:
    """The value of each E4M3 code from its sign, exponent and mantissa fields (R19)."""
    c = np.asarray(c, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64)))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


# the 256 code values, decoded once from the fields
_E4M3_VALUES = _e4m3_fields(np.arange(256))


def e4m3_to_float(codes: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3 codes (uint8) -> float64 values (R19): each code's value
    from its fields (looked up among the 256 decoded once)."""
    return _E4M3_VALUES[np.asarray(codes, dtype=np.uint8)]


def fp8_ffn_weights(cg, cu, cd, sg, su, sd, dtype=np.float64):
    """One FFN's weights from FP8 codes and per-hidden-unit scales (R20):
    cg, cu [H, F] and cd [F, H] uint8 codes; sg, su, sd [F] float32 scales.
    Returns (Wg, Wu, Wd) with each product formed in float64, then cast."""
    s = lambda v: np.asarray(v, dtype=np.float32).astype(np.float64)
    wg = e4m3_to_float(cg) * s(sg)[None, :]
    wu = e4m3_to_float(cu) * s(su)[None, :]
    wd = e4m3_to_float(cd) * s(sd)[:, None]
    return wg.astype(dtype), wu.astype(dtype), wd.astype(dtype)


def ffn_weights(W, l: int, e: int, f, dtype):
    """Expert e's (or a dense layer's, e = 0) gate, up and down matrices of
    layer l: bf16 weights through W, or FP8 codes and scales when W carries
    them (W.fp8_ffn(l, e) -> (cg, cu, cd, sg, su, sd))."""
    q = getattr(W, "fp8_ffn", None)
    if q is None:
        return f(W("wg", l, e)), f(W("wu", l, e)), f(W("wd", l, e))
    return fp8_ffn_weights(*q(l, e), dtype=dtype)


# ------------------------------------------------------------ pieces ------

def rmsnorm(h: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis (R3): h / sqrt(mean(h^2) + eps) * gamma.

    The megakernel post (section "Reduce wave quantization") fuses it with the
    residual add at the end of each parallel layer.
    """
    ms = np.mean(h * h, axis=-1, keepdims=True)
    return h / np.sqrt(ms + h.dtype.type(eps)) * gamma


def rope(x: np.ndarray, pos: int, theta: float) -> np.ndarray:
    """Rotary embedding at one position on [..., D] (R4).

    Pair i is (x[2i], x[2i+1]); it turns by angle pos * theta^(-2i/D), the
    angle and its cosine and sine formed in float64 and then cast to x's dtype
    (tiny-vllm walkthrough, section "RoPE: one current position, recomputed
    on every call"; the megakernel post applies it in the QKV epilogue,
    section "Tasks").
    """
    D = x.shape[-1]
    i = np.arange(D // 2, dtype=np.float64)
    freq = np.power(np.float64(theta), -2.0 * i / D)
    ang = np.float64(pos) * freq
    c = np.cos(ang).astype(x.dtype)
    s = np.sin(ang).astype(x.dtype)
    xe = x[..., 0::2]
    xo = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = xe * c - xo * s
    out[..., 1::2] = xe * s + xo * c
    return out


def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z / (1 + exp(-z)) (R9; the SiLU-and-multiply of section "Tasks")."""
    with np.errstate(over="ignore"):
        return z / (z.dtype.type(1) + np.exp(-z))


def softmax(v: np.ndarray) -> np.ndarray:
    """Max-subtracted softmax over the last axis."""
    m = np.max(v, axis=-1, keepdims=True)
    e = np.exp(v - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def attention_one_head(q: np.ndarray, K: np.ndarray, V: np.ndarray) -> np.ndarray:
    """softmax(K q / sqrt(D)) V for one query vector over n keys (R7).

    q [D]; K, V [n, D]. This is the attention of one decode token; the split
    into partial KV slices and their merge (megakernel post, section "Tasks",
    ATTN_DECODE / ATTN_COMBINE) must reproduce it exactly up to rounding.
    """
    D = q.shape[-1]
    s = (K @ q) / q.dtype.type(np.sqrt(D))
    p = softmax(s)
    return p @ V


def router_topk(r: np.ndarray, k: int):
    """Top-k experts of one token's router logits and their weights (R8).

    Indices in descending logit order, equal logits broken toward the lower
    expert index; weights are the softmax over the kept logits (megakernel
    post, section "Tasks": ROUTER_TOPK, and MOE_COMBINE weighting each
    expert's output by the token's router scores).
    """
    order = np.argsort(-r, kind="stable")
    idx = order[:k]
    w = softmax(r[idx])
    return idx, w


def expert_ffn(x: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray) -> np.ndarray:
    """One expert on rows x [n, H]: (silu(x Wg) * (x Wu)) Wd (R9)."""
    return (silu(x @ wg) * (x @ wu)) @ wd


def greedy(logits: np.ndarray) -> np.ndarray:
    """Argmax per row, lowest index on ties (R11); np.argmax keeps the first."""
    return np.argmax(logits, axis=-1).astype(np.int32)


# ------------------------------------------------------------ paged KV ------

def page_slot(block_table: np.ndarray, pos: np.ndarray, page_size: int):
    """(physical page, slot) of positions in one sequence (R2)."""
    pos = np.asarray(pos)
    return block_table[pos // page_size], pos % page_size


def kv_write(pool_l: np.ndarray, page: int, slot: int, g: int, k_bits: np.ndarray,
             v_bits: np.ndarray, page_size: int):
    """Store one token's K and V for group g (pool layout in mkinputs.gen):
    K plane element (slot, d) at slot*D + d; V plane at d*page_size + slot."""
    D = k_bits.shape[-1]
    pool_l[page, 0, g, slot * D:(slot + 1) * D] = k_bits
    pool_l[page, 1, g, np.arange(D) * page_size + slot] = v_bits


def kv_read(pool_l: np.ndarray, pages: np.ndarray, slots: np.ndarray, g: int, D: int,
            page_size: int, dtype):
    """K, V [n, D] of group g at the given (page, slot) pairs, as floats."""
    Kp = pool_l[:, 0, g, :].reshape(pool_l.shape[0], page_size, D)
    Vp = pool_l[:, 1, g, :].reshape(pool_l.shape[0], D, page_size)
    K = bf16_to_float(Kp[pages, slots, :], dtype)
    V = bf16_to_float(Vp[pages, :, slots], dtype)
    return K, V


# ------------------------------------------------------------ the step ------

@dataclass
class StepTrace:
    """What one step decided, per layer (lists indexed by layer)."""
    router_logits: List[np.ndarray] = field(default_factory=list)   # [B, E]
    topk_idx: List[np.ndarray] = field(default_factory=list)        # [B, k]
    topk_w: List[np.ndarray] = field(default_factory=list)          # [B, k]
    x_norm: List[np.ndarray] = field(default_factory=list)          # [B, H] (record=True)
    h_out: List[np.ndarray] = field(default_factory=list)           # [B, H] (record=True)
    q_rot: List[np.ndarray] = field(default_factory=list)           # [B, QH, D] (record=True)
    attn_out: List[np.ndarray] = field(default_factory=list)        # [B, QH*D] (record=True)
    attn_proj: List[np.ndarray] = field(default_factory=list)       # [B, H] (record=True)
    expert_out: List[np.ndarray] = field(default_factory=list)      # [B, k, H] (record=True)
    moe_out: List[np.ndarray] = field(default_factory=list)         # [B, H] (record=True; dense: the FFN's)
    h_mid: List[np.ndarray] = field(default_factory=list)           # [B, H] dense: h + attention (record=True)
    x_norm2: List[np.ndarray] = field(default_factory=list)         # [B, H] dense: the FFN's input (record=True)
    x_final: Optional[np.ndarray] = None                             # [B, H]


WeightFn = Callable[..., np.ndarray]



def _attention(cfg, W: WeightFn, pool, block_tables, seq_lens, l, x, f, dtype):
    """Layer l's attention on the normalised input x [B, H]: QKV projection,
    RoPE on q and k at each sequence's position, this step's K/V written into
    the cache (R1, R10), grouped-query attention over the cache, O projection.
    Returns (a [B, H], rotated q [B, QH, D], per-head outputs [B, QH, D])."""
    B = x.shape[0]
    H, D, P = cfg.hidden, cfg.head_dim, cfg.page_size
    QH, KVH, G = cfg.n_q_heads, cfg.n_kv_heads, cfg.group
    qkv = x @ f(W("wqkv", l))                                      # [B, QH*D + 2*KVH*D]
    q = qkv[:, :QH * D].reshape(B, QH, D)
    k = qkv[:, QH * D:QH * D + KVH * D].reshape(B, KVH, D)
    v = qkv[:, QH * D + KVH * D:].reshape(B, KVH, D)
    o = np.zeros((B, QH, D), dtype=dtype)
    qr = np.zeros((B, QH, D), dtype=dtype)
    win = cfg.layer_window(l)
    for b in range(B):
        p = int(seq_lens[b]) - 1
        qb = rope(q[b], p, cfg.rope_theta)
        qr[b] = qb
        kb = rope(k[b], p, cfg.rope_theta)
        page, slot = page_slot(block_tables[b], p, P)
        for g in range(KVH):
            kv_write(pool[l], int(page), int(slot), g, float_to_bf16_rne(kb[g]),
                     float_to_bf16_rne(v[b, g]), P)
        lo = 0 if win == 0 else max(0, p - win + 1)
        pos = np.arange(lo, p + 1)
        pages, slots = page_slot(block_tables[b], pos, P)
        for g in range(KVH):
            K, V = kv_read(pool[l], pages, slots, g, D, P, dtype)
            for hh in range(g * G, (g + 1) * G):
                o[b, hh] = attention_one_head(qb[hh], K, V)
    a = o.reshape(B, QH * D) @ f(W("wo", l))                       # [B, H]
    return a, qr, o


def _dense_layer(cfg, W: WeightFn, pool, block_tables, seq_lens, l, h, x, f, dtype, tr, record):
    """A sequential (dense) layer, as in the tiny-vllm walkthrough's
    Llama-3.2-1B decode path (section "The remaining layers and logits"): the
    attention output is added to the residual stream, a second RMSNorm
    (gamma2, the FFN's gain) normalises the sum, and the SwiGLU FFN's output
    is added in turn (megakernel post, section "Tasks": FFN_UPGATE_ACT with
    the SiLU-and-multiply, FFN_DOWN). Returns the new residual stream."""
    a, qr, o = _attention(cfg, W, pool, block_tables, seq_lens, l, x, f, dtype)
    h1 = h + a
    x2 = rmsnorm(h1, f(W("gamma2", l)), cfg.eps)
    y = expert_ffn(x2, *ffn_weights(W, l, 0, f, dtype))
    h2 = h1 + y
    if record:
        tr.x_norm.append(x)
        tr.q_rot.append(qr)
        tr.attn_out.append(o.reshape(x.shape[0], -1))
        tr.attn_proj.append(a)
        tr.h_mid.append(h1)
        tr.x_norm2.append(x2)
        tr.moe_out.append(y)
        tr.h_out.append(h2.copy())
    return h2

def decode_step(cfg, W: WeightFn, pool, block_tables: np.ndarray, tokens: np.ndarray,
                seq_lens: np.ndarray, dtype=np.float32, record: bool = False,
                router_hook=None, lm_hook=None):
    """One decode step for a batch; returns (logits [B, V] in dtype, StepTrace).

    cfg: mkinputs.configs.ModelConfig. W(name[, layer[, expert]]) returns a
    canonical weight's bf16 bits (with FP8 feed-forward weights, W.fp8_ffn
    gives their codes and scales: see ffn_weights). pool[l] is layer l's KV pool
    [n_pages, 2, KVH, page_size*D] of bf16 bits; this step's K/V are written
    into it (R1). router_hook(layer, x_norm, wr_bits) -> wr_bits, if given,
    may replace a layer's router weight before it is used, and
    lm_hook(x_final, wlm_bits) -> wlm_bits the LM head's (test inputs only:
    a hook chooses the matrices, the step's arithmetic is unchanged).
    """
    B = len(tokens)
    H, D, P = cfg.hidden, cfg.head_dim, cfg.page_size
    QH, KVH, G = cfg.n_q_heads, cfg.n_kv_heads, cfg.group
    f = lambda bits: bf16_to_float(bits, dtype)
    tr = StepTrace()

    emb = W("emb")
    h = np.stack([f(emb[int(t)]) for t in tokens])                     # [B, H]
    for l in range(cfg.n_layers):
        x = rmsnorm(h, f(W("gamma", l)), cfg.eps)                      # [B, H]
        if cfg.dense:
            h = _dense_layer(cfg, W, pool, block_tables, seq_lens, l, h, x, f, dtype, tr, record)
            continue
        # attention branch
        a, qr, o = _attention(cfg, W, pool, block_tables, seq_lens, l, x, f, dtype)
        # MoE branch
        wr = W("wr", l)
        if router_hook is not None:
            wr = router_hook(l, x, wr)
        r = x @ f(wr)                                                  # [B, E]
        idx = np.zeros((B, cfg.top_k), dtype=np.int64)
        wts = np.zeros((B, cfg.top_k), dtype=dtype)
        for b in range(B):
            idx[b], wts[b] = router_topk(r[b], cfg.top_k)
        outs = np.zeros((B, cfg.top_k, H), dtype=dtype)
        for e in np.unique(idx):
            rows, ranks = np.nonzero(idx == e)
            ye = expert_ffn(x[rows], *ffn_weights(W, l, int(e), f, dtype))
            outs[rows, ranks] = ye
        y = np.zeros((B, H), dtype=dtype)
        for j in range(cfg.top_k):
            y += wts[:, j:j + 1] * outs[:, j]
        h = h + a + y
        tr.router_logits.append(r.astype(np.float32))
        tr.topk_idx.append(idx)
        tr.topk_w.append(wts)
        if record:
            tr.x_norm.append(x)
            tr.h_out.append(h.copy())
            tr.q_rot.append(qr)
            tr.attn_out.append(o.reshape(B, QH * D))
            tr.attn_proj.append(a)
            tr.expert_out.append(outs)
            tr.moe_out.append(y)
    xf = rmsnorm(h, f(W("gamma_f")), cfg.eps)
    tr.x_final = xf
    wlm = W("wlm")
    if lm_hook is not None:
        wlm = lm_hook(xf, wlm)
    logits = xf @ f(wlm)
    return logits, tr
