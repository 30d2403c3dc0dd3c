"""Op-level GPU parity: every stage of one decode step against the oracle.

A one-layer model decodes one step over a random KV cache; the library's
scratch (read back through mk_debug_read) then holds the layer's rotated
query, attention output, O-projection partials, router logits, top-k, expert
outputs, the residual stream and the final normalised input, each compared
with the oracle's value of the same stage.
"""
import numpy as np
import pytest
import torch

from mkinputs import configs, gen
from oracle import decode as od
from tests.harness import bits_to_torch, logits_close, make_decoder, say

pytestmark = pytest.mark.gpu


# The projections run on the matrix cores with every activation operand split
# into two bf16 halves (hi = bf16(x), lo = bf16(x - hi)), so an operand carries
# a relative error near 2^-16 and a stage differs from the float32 oracle by
# float32 accumulation order plus that; the attention output is read back as
# its hi half only (one bf16 rounding, up to 2^-9 of each element, which the
# relative term covers). The other stages agree to within 1e-5 of their range.
def _close(name, got, ref, rtol=4e-3, atol_frac=3e-3):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    scale = max(np.abs(ref).max(), 1e-30)
    d = np.abs(got - ref)
    ok = np.all(d <= atol_frac * scale + rtol * np.abs(ref))
    say(f"  {name:10s} max|d|={d.max():.3e} (scale {scale:.3e}, {d.max() / scale:.1e} of it)")
    assert ok, (name, float(d.max()), scale)


def _one_layer_case(model, seq_len, seed=5, batch=1):
    wl = configs.Workload("op1", model, batch=batch, seq_len=(seq_len, seq_len))
    bs = gen.make_batch(wl, extra_steps=1)
    weights = gen.make_weights(model, seed=seed)
    pool = gen.make_kv_pool(model, bs.n_pages, seed=seed + 1)
    return wl, bs, weights, pool


@pytest.mark.parametrize("mode", [0, 1])
def test_one_layer_stages_tiny(mode):
    model = configs.small_variant(configs.TINY, n_layers=1)
    wl, bs, weights, pool = _one_layer_case(model, 40)
    say(f"[ops tiny 1-layer mode={mode}] seq_len=40")
    W = gen.NumpyWeights(weights)
    pool_np = gen.bf16_bits(pool)
    ref_pool = pool_np.copy()
    lg, tr = od.decode_step(model, W, ref_pool, bs.block_tables.numpy(), bs.tokens.numpy(),
                            bs.seq_lens.numpy(), record=True)
    pool_gpu = bits_to_torch(pool_np)
    dec = make_decoder(model, bs, pool_gpu, 41, mode)
    dec.load_weights({k: v.cuda() for k, v in weights.items()})
    logits = torch.empty((1, model.vocab), dtype=torch.float32, device="cuda")
    dec.step(bs.tokens.cuda(), bs.block_tables.cuda(), bs.seq_lens.cuda(), 40, logits)
    dec.sync()
    H, QD, KVH, K = model.hidden, model.q_dim, model.n_kv_heads, model.top_k
    _close("q", dec.debug_read("q", (1, QD)), tr.q_rot[0].reshape(1, QD))
    # the attention output is kept in bf16 (the O projection's operand)
    _close("attn o", od.bf16_to_float(dec.debug_read("o", (1, QD), "uint16")), tr.attn_out[0])
    ao = dec.debug_read("ao", (KVH, 1, H))
    _close("o-proj", ao.sum(0), tr.attn_proj[0])
    # router partial sums over K halves (hidden < 1024) or quarters
    n_ks = 2 if H < 1024 else 4
    rp = dec.debug_read("rp", (n_ks, 1, model.n_experts))
    _close("router", rp.sum(0), tr.router_logits[0])
    idx = dec.debug_read("tk_idx", (1, K), "int32")
    assert sorted(idx[0].tolist()) == sorted(tr.topk_idx[0][0].tolist())
    # one token runs the fused MoE: no per-expert rows, so the combined expert
    # output is checked (the block's new residual less its input and the
    # attention projection)
    h_out = dec.debug_read("h", (1, H))
    h_in = od.bf16_to_float(W("emb")[int(bs.tokens[0])], np.float64)
    _close("experts", h_out[0] - h_in - ao.sum(0)[0], tr.moe_out[0][0])
    _close("h", h_out, tr.h_out[0])
    ok, mx, rl2 = logits_close(logits.cpu().numpy()[0], lg[0])
    say(f"  logits max|d|={mx:.2e} relL2={rl2:.2e}")
    assert ok
    dec.close()
