"""GPU parity at full size, in the launch configuration bench.py times.

The shapes are the full model's (hidden 2048, 32 query / 4 kv heads of 128,
128 experts top-8 of width 768, vocab 131072) with random bf16 weights drawn
on the GPU exactly as bench.py draws them, over an 8K context of synthetic
N(0, 1) K/V:

- the one-layer model: three teacher-forced steps in both modes, every
  stage of the first step (rotated query, attention output, O-projection
  partials, router logits, top-k, expert outputs, residual) and every step's
  logits, greedy token, top-k set and appended K/V; the same model at a
  262144-token context, at batch 4 with 64K contexts and at batch 32 with
  ragged 512..16384 contexts;
- the 48-layer model (12 full, 36 window-4096 layers) in the megakernel:
  eight greedy steps at batch 1 and 8K with the kernel advancing tokens and
  lengths itself; two steps at batch 32 with ragged 512..16384 contexts
  (window and full layers, the claiming MoE at every layer); batch 1 at
  262144 positions and batch 4 at 65536: logits, greedy tokens and all 48
  layers' top-k sets of every row and step.

The oracle runs on the host with the same weights. Before a step is compared,
oracle hooks widen any token's gap between its 8th and 9th router logit, and
any row's gap between its two largest logits, to 2e-2 by moving whole bf16
steps of the two router (LM-head) columns involved; the GPU receives the same
repaired matrices, so every top-k set and greedy token is decided by a margin
far above the bf16 operand rounding (about 1e-3 on these logits) and every
one of them is compared.
"""
import numpy as np
import pytest
import torch

from mkinputs import configs, gen
from oracle import decode as od
from oracle import trajectory as tj
from tests.harness import (RepairUploads, bits_to_torch, lm_repair_hook, logits_close, make_decoder,
                           router_repair_hook, say, torch_to_bits)

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]


class FullCase:
    def __init__(self, wl, steps, mode, fp8=False):
        m = wl.model
        self.wl, self.m, self.steps, self.fp8 = wl, m, steps, fp8
        dev = torch.device("cuda:0")
        self.bs = gen.make_batch(wl, extra_steps=steps)
        self.pool = gen.make_kv_pool(m, self.bs.n_pages, seed=wl.seed_kv, device=dev)
        self.pool_host = gen.bf16_bits(self.pool)
        self.pool0 = self.pool_host.copy()
        self.dec = make_decoder(m, self.bs, self.pool, int(self.bs.seq_lens.max()) + steps, mode, ffn_fp8=fp8)
        hook, self.repaired = router_repair_hook(m)
        n_layers = m.n_layers

        def router_hook(l, x, wr):  # (progress on long oracle steps)
            if l % 12 == 11 or l == n_layers - 1:
                say(f"    oracle at layer {l}")
            return hook(l, x, wr)

        self.hook = router_hook
        self.lm_hook, self.lm_state = lm_repair_hook()
        g = {n: gen.weight_tensor(m, n, wl.seed_weights, dev) for n in gen.GLOBAL_NAMES}
        self.dec.load_globals(g["emb"], g["gamma_f"], g["wlm"])
        del g
        for l in range(m.n_layers):
            self._load_layer(l)
        torch.cuda.synchronize()
        self.W = gen.LazyWeights(m, wl.seed_weights, device="cuda", fp8=fp8)
        self.up = RepairUploads(self.dec, self.repaired, self.lm_state,
                                lambda l: gen.make_layer_weights(m, l, wl.seed_weights, "cuda"),
                                lambda: {n: gen.weight_tensor(m, n, wl.seed_weights, dev) for n in gen.GLOBAL_NAMES})
        self.bt = self.bs.block_tables.cuda()
        B = wl.batch
        self.route = torch.full((m.n_layers, B, m.top_k), -1, dtype=torch.int32, device=dev)
        self.dec.set_routing_trace(self.route)
        self.logits = torch.empty((B, m.vocab), dtype=torch.float32, device=dev)
        self.nxt = torch.empty(B, dtype=torch.int32, device=dev)

    def _load_layer(self, l):
        w = gen.make_layer_weights(self.m, l, self.wl.seed_weights, "cuda")
        if l in self.repaired:
            w[f"wr.{l}"] = bits_to_torch(self.repaired[l])
        if self.fp8:
            q = gen.quantize_ffn_fp8(w.pop(f"wg.{l}"), w.pop(f"wu.{l}"), w.pop(f"wd.{l}"))
            self.dec.load_ffn_fp8(l, *q)
        self.dec.load_layer(l, *(w.get(f"{k}.{l}") for k in gen.layer_kinds(self.m)))
        torch.cuda.synchronize()

    def oracle_step(self, tokens, lens, record=True):
        lg, tr = od.decode_step(self.m, self.W, self.pool_host, self.bs.block_tables.numpy(), tokens, lens,
                                record=record, router_hook=self.hook, lm_hook=self.lm_hook)
        # the GPU gets every router and LM-head matrix the hooks changed
        self.up.sync()
        return lg, tr

    def gpu_step(self, tokens, lens, advance=False):
        if advance:  # the kernel's own tokens and lengths (device tensors)
            self.dec.step(tokens, self.bt, lens, int(lens.max().item()), self.logits, self.nxt, advance=True)
        else:
            self.dec.step(torch.tensor(tokens, dtype=torch.int32, device="cuda"), self.bt,
                          torch.tensor(lens, dtype=torch.int32, device="cuda"), int(lens.max()), self.logits,
                          self.nxt)
        self.dec.sync()
        return self.logits.cpu().numpy(), self.nxt.cpu().numpy(), self.route.cpu().numpy()

    def compare(self, s, lg_ref, tr_ref, lg, tok, route):
        ref_tok = od.greedy(lg_ref)
        gaps = tj.greedy_gap(lg_ref)
        worst = (0.0, 0.0)
        for b in range(lg.shape[0]):
            ok, mx, rl2 = logits_close(lg[b], lg_ref[b])
            worst = (max(worst[0], mx), max(worst[1], rl2))
            if lg.shape[0] <= 4:
                say(f"  step {s} row {b}: logits max|d|={mx:.2e} relL2={rl2:.2e}; token gpu={int(tok[b])} "
                    f"ref={int(ref_tok[b])} (gap {gaps[b]:.3f})")
            assert ok, (s, b, mx, rl2)
            assert int(tok[b]) == int(ref_tok[b]), (s, b, float(gaps[b]))
            for l in range(0 if self.m.dense else self.m.n_layers):  # (a dense model routes nothing)
                assert sorted(route[l, b].tolist()) == sorted(tr_ref.topk_idx[l][b].tolist()), (s, b, l)
        say(f"  step {s}: {lg.shape[0]} rows, worst logits max|d|={worst[0]:.2e} relL2={worst[1]:.2e}, every "
            f"greedy token{'' if self.m.dense else f' and {self.m.n_layers} layers top-k'} equal; repaired router "
            f"layers {len(self.repaired)}, LM-head repairs {self.lm_state['repairs']}")

    def check_kv(self, lens_per_step):
        gpu = torch_to_bits(self.pool)
        m, P = self.m, self.m.page_size
        touched = np.zeros(gpu.shape, bool)
        for lens in lens_per_step:
            for b in range(len(lens)):
                pos = int(lens[b]) - 1
                page = int(self.bs.block_tables[b, pos // P])
                for plane in range(2):
                    a = od.bf16_to_float(gpu[:, page, plane], np.float64)
                    r = od.bf16_to_float(self.pool_host[:, page, plane], np.float64)
                    t = touched[:, page, plane]
                    if plane == 0:
                        shape, sel = (m.n_layers, m.n_kv_heads, P, m.head_dim), (slice(None), slice(None), pos % P)
                    else:
                        shape, sel = (m.n_layers, m.n_kv_heads, m.head_dim, P), (Ellipsis, pos % P)
                    a, r = a.reshape(shape)[sel], r.reshape(shape)[sel]
                    t.reshape(shape)[sel] = True
                    for l in range(m.n_layers):
                        d = np.abs(a[l] - r[l])
                        assert d.max() <= 1e-2 * np.abs(r[l]).max() + 1e-3, (pos, l, plane, float(d.max()))
        assert np.array_equal(gpu[~touched], self.pool0[~touched]), "a slot no step appended to changed"

    def close(self):
        self.dec.close()
        torch.cuda.empty_cache()


def _stages_layer1(c, tr):
    """Every stage of the one-layer model's step against the oracle's trace."""
    m, d = c.m, c.dec
    H, QD, KVH, K = m.hidden, m.q_dim, m.n_kv_heads, m.top_k

    # (split-bf16 operands: stages agree to well under 0.1% of their range;
    # the attention output is read back as its bf16 hi half)
    def close(name, got, ref, rtol=4e-3, atol_frac=3e-3):
        got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
        scale = max(np.abs(ref).max(), 1e-30)
        dd = np.abs(got - ref)
        say(f"    {name:10s} max|d|={dd.max():.3e} (scale {scale:.3e}, {dd.max() / scale:.1e} of it)")
        assert np.all(dd <= atol_frac * scale + rtol * np.abs(ref)), name

    close("q", d.debug_read("q", (1, QD)), tr.q_rot[0].reshape(1, QD))
    close("attn o", od.bf16_to_float(d.debug_read("o", (1, QD), "uint16")), tr.attn_out[0])
    close("o-proj", d.debug_read("ao", (KVH, 1, H)).sum(0), tr.attn_proj[0])
    rp = d.debug_read("rp", (4, 1, m.n_experts))
    close("router", rp.sum(0), tr.router_logits[0])
    idx = d.debug_read("tk_idx", (1, K), "int32")
    assert sorted(idx[0].tolist()) == sorted(tr.topk_idx[0][0].tolist())
    # one token runs the fused MoE (no per-expert rows): the combined expert
    # output, from the new residual less its input and the attention projection
    h_out = d.debug_read("h", (1, H))
    h_in = od.bf16_to_float(c.W("emb")[int(c.bs.tokens[0])], np.float64)
    ao = d.debug_read("ao", (KVH, 1, H)).sum(0)
    close("experts", h_out[0] - h_in - ao[0], tr.moe_out[0][0])
    close("h", h_out, tr.h_out[0])


def _run(wl, steps, mode, stages, advance=False, fp8=False):
    say(f"[full {wl.name} mode={mode}{' fp8' if fp8 else ''}] {steps} steps from seq_len {wl.seq_len[0]}"
        f"{' (in-kernel advance)' if advance else ''}")
    c = FullCase(wl, steps, mode, fp8)
    try:
        tokens = c.bs.tokens.numpy().copy()
        lens = c.bs.seq_lens.numpy().astype(np.int64)
        tok_dev = torch.tensor(tokens, dtype=torch.int32, device="cuda")
        lens_dev = torch.tensor(lens, dtype=torch.int32, device="cuda")
        seen = []
        for s in range(steps):
            lg_ref, tr_ref = c.oracle_step(tokens, lens, record=stages and s == 0)
            if advance:
                # the kernel fed itself: its input must be the oracle's
                assert np.array_equal(tok_dev.cpu().numpy(), tokens) and np.array_equal(lens_dev.cpu().numpy(), lens)
                lg, tok, route = c.gpu_step(tok_dev, lens_dev, advance=True)
            else:
                lg, tok, route = c.gpu_step(tokens, lens)
            if stages and s == 0:
                _stages_layer1(c, tr_ref)
            c.compare(s, lg_ref, tr_ref, lg, tok, route)
            seen.append(lens.copy())
            tokens = od.greedy(lg_ref)
            lens = lens + 1
        c.check_kv(seen)
    finally:
        c.close()


@pytest.mark.parametrize("mode", [0, 1])
def test_layer1_b1_8k(mode):
    _run(configs.WORKLOADS["layer1_b1_8k"], 3, mode, stages=True)


@pytest.mark.parametrize("name", ["layer1_b1_256k", "layer1_b4_64k", "layer1_b32_ragged"])
def test_layer1_long_and_batched(name):
    """The split-KV attention over 256K positions (more than 250 splits
    merged), four 64K sequences, and 32 ragged sequences (two row tiles)."""
    _run(configs.WORKLOADS[name], 2, 0, stages=False)


def test_full48_b1_8k_megakernel():
    """Eight greedy steps of the benchmark configuration, the kernel writing
    each step's token and length for the next (as bench.py runs it)."""
    _run(configs.WORKLOADS["full48_b1_8k"], 8, 0, stages=False, advance=True)


def test_full48_b32_ragged_megakernel():
    """Batch 32, ragged 512..16384 contexts: window layers with rows on both
    sides of the window, the claiming MoE at every layer, two row tiles."""
    _run(configs.WORKLOADS["full48_b32_ragged"], 2, 0, stages=False)


@pytest.mark.parametrize("name", ["full48_b1_256k", "full48_b4_64k"])
def test_full48_long_context_megakernel(name):
    """The long-context workloads: full layers split over every compute unit."""
    _run(configs.WORKLOADS[name], 1, 0, stages=False)
