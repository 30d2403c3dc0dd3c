"""Pins of the oracle to things other than itself (CPU only).

Each test fixes part of the oracle against a closed form, an invariant, a
library routine for a special case, brute force on tiny inputs, or an
independent full-sequence recomputation, chosen so that a plausible mistake
(a dropped term, a wrong sign or index, a transposed operand, a wrong pairing
or position) fails at least one of them.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

from mkinputs import configs, gen
from oracle import decode as od


# ------------------------------------------------------------------ bf16 ----

def test_bf16_known_patterns():
    vals = np.array([1.0, -2.0, 0.1, 1.00390625, 1.01171875, 3.0e38, 1e-40], dtype=np.float32)
    # 0.1 = 0x3DCCCCCD rounds up; 1.00390625 = 0x3F808000 is a tie to even (down);
    # 1.01171875 = 0x3F818000 is a tie with odd upper half (up).
    want = [0x3F80, 0xC000, 0x3DCD, 0x3F80, 0x3F82]
    got = od.float_to_bf16_rne(vals)
    assert list(got[:5]) == want
    # agrees with torch's conversion (RNE) on random values incl. subnormals
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-90, 80, 100000))).astype(np.float32)
    t = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(od.float_to_bf16_rne(x), t)
    assert np.array_equal(od.bf16_to_float(t), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


# --------------------------------------------------------------- RMSNorm ----

def test_rmsnorm_closed_form():
    h = np.array([[3.0, 4.0]])
    g = np.array([2.0, 0.5])
    out = od.rmsnorm(h, g, 0.0)
    r = math.sqrt((9 + 16) / 2)
    assert np.allclose(out, [[2 * 3 / r, 0.5 * 4 / r]], rtol=1e-15)
    # eps enters under the root
    out = od.rmsnorm(h, np.ones(2), 0.5)
    assert np.allclose(out, h / math.sqrt(12.5 + 0.5), rtol=1e-15)


def test_rmsnorm_unit_rms_and_scale_invariance():
    rng = np.random.default_rng(1)
    h = rng.standard_normal((3, 2048))
    out = od.rmsnorm(h, np.ones(2048), 1e-6)
    rms = np.sqrt(np.mean(out ** 2, axis=-1))
    ms = np.mean(h ** 2, axis=-1)
    assert np.allclose(rms, np.sqrt(ms / (ms + 1e-6)), rtol=1e-12)
    assert np.allclose(od.rmsnorm(7.5 * h, np.ones(2048), 0.0), od.rmsnorm(h, np.ones(2048), 0.0), rtol=1e-12)


# ------------------------------------------------------------------ RoPE ----

def test_rope_identity_at_zero_and_pair_layout():
    D = 128
    rng = np.random.default_rng(2)
    x = rng.standard_normal(D)
    assert np.allclose(od.rope(x, 0, 1e4), x, rtol=0, atol=0)
    p = 37
    for i in (0, 1, 5, 63):
        f = 1e4 ** (-2 * i / D)
        e = np.zeros(D); e[2 * i] = 1.0
        out = od.rope(e, p, 1e4)
        assert math.isclose(out[2 * i], math.cos(p * f), abs_tol=1e-15)
        assert math.isclose(out[2 * i + 1], math.sin(p * f), abs_tol=1e-15)
        assert np.count_nonzero(out) <= 2
        e = np.zeros(D); e[2 * i + 1] = 1.0
        out = od.rope(e, p, 1e4)
        assert math.isclose(out[2 * i], -math.sin(p * f), abs_tol=1e-15)
        assert math.isclose(out[2 * i + 1], math.cos(p * f), abs_tol=1e-15)


def test_rope_complex_form_and_relative_property():
    D = 64
    rng = np.random.default_rng(3)
    q = rng.standard_normal(D)
    k = rng.standard_normal(D)
    # complex rotation: (x0 + i x1) * exp(i p f)
    p = 1234
    f = 1e4 ** (-np.arange(D // 2) * 2.0 / D)
    z = (q[0::2] + 1j * q[1::2]) * np.exp(1j * p * f)
    out = od.rope(q, p, 1e4)
    assert np.allclose(out[0::2], z.real, atol=1e-12) and np.allclose(out[1::2], z.imag, atol=1e-12)
    # per-pair norms preserved
    assert np.allclose(np.hypot(out[0::2], out[1::2]), np.hypot(q[0::2], q[1::2]), rtol=1e-13)
    # scores depend only on the position difference
    s1 = od.rope(q, 100, 1e4) @ od.rope(k, 40, 1e4)
    s2 = od.rope(q, 5100, 1e4) @ od.rope(k, 5040, 1e4)
    assert abs(s1 - s2) < 1e-9


def test_rope_large_position_uses_float64_angle():
    # at p = 262143 a float32 angle would be off by ~1e-2 rad; the oracle's is exact
    D = 128
    e = np.zeros(D, dtype=np.float32); e[0] = 1.0
    out = od.rope(e, 262143, 1e4)
    assert abs(out[0] - math.cos(262143.0)) < 1e-6 and abs(out[1] - math.sin(262143.0)) < 1e-6


# ------------------------------------------------------------------ SiLU ----

def test_silu_closed_forms():
    z = np.array([0.0, 1.0, -1.0, 40.0, -100.0, -1000.0])
    out = od.silu(z)
    assert out[0] == 0.0
    assert math.isclose(out[1], 1 / (1 + math.exp(-1)), rel_tol=1e-15)
    assert math.isclose(out[2], -1 / (1 + math.e), rel_tol=1e-15)
    assert math.isclose(out[3], 40.0, rel_tol=1e-15)
    assert abs(out[4]) < 1e-40 and out[5] == 0.0
    # library special case: silu(z) = z * expit(z)
    zz = np.linspace(-20, 20, 1001)
    assert np.allclose(od.silu(zz), zz * scipy.special.expit(zz), rtol=1e-14, atol=1e-300)


# ------------------------------------------------------------- attention ----

def test_attention_special_cases():
    rng = np.random.default_rng(4)
    D = 16
    q = rng.standard_normal(D)
    V = rng.standard_normal((5, D))
    # one key: output is that value
    assert np.allclose(od.attention_one_head(q, rng.standard_normal((1, D)), V[:1]), V[0], rtol=1e-15)
    # zero query: uniform weights -> mean of values
    assert np.allclose(od.attention_one_head(np.zeros(D), rng.standard_normal((5, D)), V), V.mean(0), rtol=1e-14)
    # one dominant key picks its value
    K = rng.standard_normal((5, D)) * 0.01
    K[3] = q * 1000
    assert np.allclose(od.attention_one_head(q, K, V), V[3], atol=1e-12)


def test_attention_matches_library_softmax_and_brute_force():
    rng = np.random.default_rng(5)
    D, n = 8, 7
    q, K, V = rng.standard_normal(D), rng.standard_normal((n, D)), rng.standard_normal((n, D))
    ref = scipy.special.softmax(K @ q / math.sqrt(D)) @ V
    assert np.allclose(od.attention_one_head(q, K, V), ref, rtol=1e-13)
    # brute force with math.exp, no max subtraction
    w = [math.exp(sum(q[d] * K[j, d] for d in range(D)) / math.sqrt(D)) for j in range(n)]
    bf = [sum(w[j] * V[j, d] for j in range(n)) / sum(w) for d in range(D)]
    assert np.allclose(od.attention_one_head(q, K, V), bf, rtol=1e-12)
    # permuting keys together with values changes nothing
    perm = rng.permutation(n)
    assert np.allclose(od.attention_one_head(q, K[perm], V[perm]), ref, rtol=1e-13)


# ---------------------------------------------------------------- router ----

def test_router_topk_ties_order_and_weights():
    r = np.array([1.0, 3.0, 3.0, 2.0, 3.0])
    idx, w = od.router_topk(r, 2)
    assert list(idx) == [1, 2]
    assert np.allclose(w, [0.5, 0.5])
    idx, w = od.router_topk(r, 4)
    assert list(idx) == [1, 2, 4, 3]
    rng = np.random.default_rng(6)
    r = rng.standard_normal(128).astype(np.float32)
    idx, w = od.router_topk(r, 8)
    assert len(set(idx.tolist())) == 8
    assert np.all(np.diff(r[idx]) <= 0)
    assert set(idx.tolist()) == set(np.argsort(r)[::-1][:8].tolist())
    assert abs(float(w.sum()) - 1.0) <= 1e-6 and np.all(w > 0)
    # k = E reduces to the dense softmax (library routine)
    idx, w = od.router_topk(r.astype(np.float64), 128)
    dense = scipy.special.softmax(r.astype(np.float64))
    assert np.allclose(w, dense[idx], rtol=1e-13)
    # renormalised softmax: full softmax restricted to the top-k, rescaled
    idx, w = od.router_topk(r.astype(np.float64), 8)
    assert np.allclose(w, dense[idx] / dense[idx].sum(), rtol=1e-12)


def test_greedy_lowest_index_on_ties():
    lg = np.array([[0.5, 2.0, 2.0, 1.0], [3.0, 3.0, 3.0, 3.0]], dtype=np.float32)
    assert list(od.greedy(lg)) == [1, 0]


# ---------------------------------------------------------------- expert ----

def test_expert_ffn_brute_force():
    rng = np.random.default_rng(7)
    H, F = 6, 4
    x = rng.standard_normal((2, H))
    wg, wu, wd = rng.standard_normal((H, F)), rng.standard_normal((H, F)), rng.standard_normal((F, H))
    out = od.expert_ffn(x, wg, wu, wd)
    for b in range(2):
        for o in range(H):
            acc = 0.0
            for f in range(F):
                g = sum(x[b, i] * wg[i, f] for i in range(H))
                u = sum(x[b, i] * wu[i, f] for i in range(H))
                acc += g / (1 + math.exp(-g)) * u * wd[f, o]
            assert math.isclose(out[b, o], acc, rel_tol=1e-12, abs_tol=1e-12)


# ------------------------------------------------------- whole-step pins ----

def _tiny(window=0, full_every=1, layers=2):
    return configs.small_variant(configs.TINY, window=window, full_every=full_every, n_layers=layers)


def _weights(cfg, seed=11):
    return gen.NumpyWeights(gen.make_weights(cfg, seed=seed, device="cpu"))


def _empty_pool(cfg, n_pages):
    return np.zeros(gen.kv_pool_shape(cfg, n_pages), dtype=np.uint16)


def _run_incremental(cfg, W, toks, bt, dtype):
    pool = _empty_pool(cfg, bt.max() + 1)
    outs, traces = [], []
    for t, tok in enumerate(toks):
        lg, tr = od.decode_step(cfg, W, pool, bt[None, :], np.array([tok]), np.array([t + 1]), dtype=dtype)
        outs.append(lg[0]); traces.append(tr)
    return np.array(outs), traces, pool


def _full_sequence_forward(cfg, W, toks):
    """Prefill-style forward of a whole sequence, float64, written independently
    of the oracle: matrix form over positions, complex-number RoPE, explicit
    causal/window masks, scipy softmax, K/V rounded to bf16 like the cache."""
    f = lambda a: gen.torch.from_numpy(a.view(np.int16).copy()).view(gen.torch.bfloat16).double().numpy()
    T, H, D = len(toks), cfg.hidden, cfg.head_dim
    QH, KVH = cfg.n_q_heads, cfg.n_kv_heads
    rb = lambda a: gen.torch.from_numpy(np.asarray(a, dtype=np.float32)).to(gen.torch.bfloat16).double().numpy()
    h = f(W("emb"))[np.asarray(toks)]
    pos = np.arange(T)
    freqs = cfg.rope_theta ** (-np.arange(D // 2) * 2.0 / D)
    rot = np.exp(1j * pos[:, None] * freqs[None, :])                     # [T, D/2]

    def rms(v, g):
        return v / np.sqrt((np.linalg.norm(v, axis=-1, keepdims=True) ** 2) / v.shape[-1] + cfg.eps) * g

    def rope_all(v):                                                      # [T, n, D]
        z = (v[..., 0::2] + 1j * v[..., 1::2]) * rot[:, None, :]
        out = np.empty_like(v); out[..., 0::2] = z.real; out[..., 1::2] = z.imag
        return out

    for l in range(cfg.n_layers):
        x = rms(h, f(W("gamma", l)))
        qkv = x @ f(W("wqkv", l))
        q = rope_all(qkv[:, :QH * D].reshape(T, QH, D))
        k = rb(rope_all(qkv[:, QH * D:(QH + KVH) * D].reshape(T, KVH, D)))
        v = rb(qkv[:, (QH + KVH) * D:].reshape(T, KVH, D))
        win = cfg.layer_window(l)
        allowed = pos[None, :] <= pos[:, None]
        if win:
            allowed &= pos[None, :] > pos[:, None] - win
        o = np.zeros((T, QH, D))
        for hh in range(QH):
            g = hh * KVH // QH
            s = q[:, hh] @ k[:, g].T / math.sqrt(D)
            s = np.where(allowed, s, -np.inf)
            o[:, hh] = scipy.special.softmax(s, axis=-1) @ v[:, g]
        a = o.reshape(T, QH * D) @ f(W("wo", l))
        if cfg.dense:
            # sequential: the FFN reads the second norm of h + attention
            h = h + a
            x2 = rms(h, f(W("gamma2", l)))
            g_ = x2 @ f(W("wg", l, 0))
            u_ = x2 @ f(W("wu", l, 0))
            h = h + (g_ * scipy.special.expit(g_) * u_) @ f(W("wd", l, 0))
            continue
        r = x @ f(W("wr", l))
        y = np.zeros((T, H))
        for t in range(T):
            order = np.lexsort((np.arange(cfg.n_experts), -r[t]))[:cfg.top_k]
            wts = scipy.special.softmax(r[t, order])
            for j, e in enumerate(order):
                g_ = x[t] @ f(W("wg", l, int(e)))
                u_ = x[t] @ f(W("wu", l, int(e)))
                y[t] += wts[j] * ((g_ * scipy.special.expit(g_) * u_) @ f(W("wd", l, int(e))))
        h = h + a + y
    return rms(h, f(W("gamma_f"))) @ f(W("wlm"))


@pytest.mark.parametrize("window,full_every", [(0, 1), (8, 2)])
def test_incremental_decode_matches_full_recomputation(window, full_every):
    cfg = _tiny(window=window, full_every=full_every)
    W = _weights(cfg)
    rng = np.random.default_rng(8)
    T = 37                                 # crosses two page boundaries, ragged last page
    toks = rng.integers(0, cfg.vocab, T)
    bt = rng.permutation(8)[:3]            # scattered pages
    inc, _, _ = _run_incremental(cfg, W, toks, bt, np.float64)
    full = _full_sequence_forward(cfg, W, toks)
    assert np.max(np.abs(inc - full)) < 1e-9


def test_dense_incremental_decode_matches_full_recomputation():
    """The dense sequential layer (attention added, a second norm, the SwiGLU
    FFN added) step by step equals the whole-sequence float64 forward."""
    cfg = configs.TINY_DENSE
    W = _weights(cfg)
    rng = np.random.default_rng(18)
    T = 37
    toks = rng.integers(0, cfg.vocab, T)
    bt = rng.permutation(8)[:3]
    inc, _, _ = _run_incremental(cfg, W, toks, bt, np.float64)
    full = _full_sequence_forward(cfg, W, toks)
    assert np.max(np.abs(inc - full)) < 1e-9


def test_dense_layer_with_silent_outputs_keeps_the_embedding():
    """With the O projection and the FFN's down projection zero, every dense
    layer adds nothing: the logits are RMSNorm(emb[token]; gamma_f) times the
    tied head (the embedding transposed), whatever the attention and the
    norms inside the layer compute."""
    cfg = configs.TINY_DENSE
    t = gen.make_weights(cfg, seed=12, device="cpu")
    for l in range(cfg.n_layers):
        t[f"wo.{l}"] = gen.torch.zeros_like(t[f"wo.{l}"])
        t[f"wd.{l}"] = gen.torch.zeros_like(t[f"wd.{l}"])
    W = gen.NumpyWeights(t)
    toks = np.array([5, 900])
    pool = _empty_pool(cfg, 4)
    lg, _ = od.decode_step(cfg, W, pool, np.array([[0], [1]]), toks, np.array([1, 1]), dtype=np.float64)
    emb = t["emb"].double().numpy()
    gf = t["gamma_f"].double().numpy()
    for b, tok in enumerate(toks):
        e = emb[tok]
        x = e / math.sqrt(float(np.mean(e * e)) + cfg.eps) * gf
        assert np.max(np.abs(lg[b] - emb @ x)) < 1e-10


def test_dense_head_is_the_embedding_transposed():
    cfg = configs.TINY_DENSE
    W = _weights(cfg)
    assert np.array_equal(W("wlm"), W("emb").T)
    assert "wr.0" not in gen.weight_shapes(cfg) and gen.weight_shapes(cfg)["gamma2.1"] == (cfg.hidden,)


def test_paged_equals_contiguous_bit_identical():
    cfg = _tiny()
    W = _weights(cfg)
    rng = np.random.default_rng(9)
    toks = rng.integers(0, cfg.vocab, 40)
    a, _, pa = _run_incremental(cfg, W, toks, np.array([0, 1, 2]), np.float32)
    b, _, pb = _run_incremental(cfg, W, toks, np.array([6, 2, 4]), np.float32)
    assert np.array_equal(a, b)
    assert np.array_equal(pa[:, [0, 1, 2]], pb[:, [6, 2, 4]])


def test_float32_oracle_tracks_float64():
    cfg = _tiny()
    W = _weights(cfg)
    rng = np.random.default_rng(10)
    toks = rng.integers(0, cfg.vocab, 20)
    bt = np.array([3, 1])
    a, _, _ = _run_incremental(cfg, W, toks, bt, np.float32)
    b, _, _ = _run_incremental(cfg, W, toks, bt, np.float64)
    assert np.max(np.abs(a - b)) < 1e-4


def test_batch_rows_are_independent():
    """A batched step equals the per-sequence steps (same weights, own caches)."""
    cfg = _tiny()
    W = _weights(cfg)
    rng = np.random.default_rng(12)
    pool = od.float_to_bf16_rne(rng.standard_normal(gen.kv_pool_shape(cfg, 12)).astype(np.float32))
    bt = np.array([[0, 5, 7, -1], [2, 3, 11, 9], [1, 4, -1, -1]])
    lens = np.array([40, 64, 17])
    toks = np.array([5, 900, 17])
    p1 = pool.copy()
    lg, _ = od.decode_step(cfg, W, p1, bt, toks, lens, dtype=np.float64)
    for b in range(3):
        p2 = pool.copy()
        lb, _ = od.decode_step(cfg, W, p2, bt[b:b + 1], toks[b:b + 1], lens[b:b + 1], dtype=np.float64)
        assert np.allclose(lb[0], lg[b], rtol=0, atol=1e-12)


def test_moe_reduces_to_single_ffn_when_experts_identical():
    """All experts equal -> the weighted mixture is that one FFN (weights sum to 1)."""
    cfg = _tiny(layers=1)
    ws = gen.make_weights(cfg, seed=13, device="cpu")
    for nm in ("wg.0", "wu.0", "wd.0"):
        ws[nm][:] = ws[nm][0:1].clone()
    W = gen.NumpyWeights(ws)
    rng = np.random.default_rng(14)
    pool = np.zeros(gen.kv_pool_shape(cfg, 2), dtype=np.uint16)
    lg, tr = od.decode_step(cfg, W, pool, np.array([[0, 1]]), np.array([7]), np.array([1]),
                            dtype=np.float64, record=True)
    x = tr.x_norm[0]
    f = lambda a: od.bf16_to_float(a, np.float64)
    ffn = od.expert_ffn(x, f(W("wg", 0, 0)), f(W("wu", 0, 0)), f(W("wd", 0, 0)))
    # recompute h from the pieces with a single FFN: h1 - ffn must equal h0 + attention part
    h0 = f(W("emb"))[7]
    h1 = tr.h_out[0][0]
    attn_part = h1 - h0 - ffn[0]
    # attention at seq_len 1 returns v, so the attention part is v_rep @ Wo
    qkv = x @ f(W("wqkv", 0))
    D, QH, KVH = cfg.head_dim, cfg.n_q_heads, cfg.n_kv_heads
    v = od.bf16_to_float(od.float_to_bf16_rne(qkv[0, (QH + KVH) * D:].astype(np.float32)), np.float64).reshape(KVH, D)
    o = np.concatenate([v[hh * KVH // QH] for hh in range(QH)])
    assert np.allclose(attn_part, o @ f(W("wo", 0)), atol=1e-10)


# ------------------------------------------------------ trajectory pins ----
# Multi-step decoding (oracle/trajectory.py) against the independent float64
# full-sequence forward above: decoding token after token with lengths + 1
# must give, at every step, the row of the whole sequence's prefill-style
# logits at that position; greedy decoding must feed each row's argmax as the
# next token.

from oracle import trajectory as tj


def test_greedy_decode_matches_full_sequence_forward():
    cfg = _tiny(window=8, full_every=2)
    W = _weights(cfg, seed=21)
    bt = np.array([[5, 2, 7]])
    pool = _empty_pool(cfg, 8)
    run = tj.greedy_decode(cfg, W, pool, bt, np.array([11]), np.array([1]), 19, dtype=np.float64)
    seq = [11] + [int(g[0]) for g in run.greedy[:-1]]
    # the tokens fed are the start token then each step's greedy choice
    assert [int(t[0]) for t in run.tokens_in] == seq
    # lengths grow by one per step from the start length
    assert [int(s[0]) for s in run.seq_lens] == list(range(1, 20))
    full = _full_sequence_forward(cfg, W, seq)
    got = np.array([lg[0] for lg in run.logits])
    assert np.max(np.abs(got - full)) < 1e-9
    # each greedy token is the full forward's argmax (lowest index on ties)
    assert [int(g[0]) for g in run.greedy] == [int(np.argmax(r)) for r in full]
    # and every step appended its K/V: 19 positions over pages 5, 2 (16 + 3)
    assert np.count_nonzero(pool[:, 5]) > 0 and np.count_nonzero(pool[:, 2]) > 0
    assert np.count_nonzero(pool[:, 7]) == 0


def test_teacher_forced_matches_full_sequence_forward_batched():
    cfg = _tiny()
    W = _weights(cfg, seed=22)
    rng = np.random.default_rng(23)
    T, B = 12, 2
    toks = rng.integers(0, cfg.vocab, (T, B))
    bt = np.array([[0, 3], [1, 2]])
    pool = _empty_pool(cfg, 4)
    run = tj.teacher_forced(cfg, W, pool, bt, toks, np.array([1, 1]), dtype=np.float64)
    assert [s.tolist() for s in run.seq_lens] == [[t + 1, t + 1] for t in range(T)]
    for b in range(B):
        full = _full_sequence_forward(cfg, W, toks[:, b])
        got = np.array([lg[b] for lg in run.logits])
        assert np.max(np.abs(got - full)) < 1e-9
        assert [int(g[b]) for g in run.greedy] == [int(np.argmax(r)) for r in full]


def test_gap_helpers_on_hand_built_rows():
    # greedy gap: largest minus second largest; a tie gives 0
    lg = np.array([[1.0, 3.0, 2.5, 3.0], [5.0, 1.0, 4.25, -2.0], [0.0, 0.0, 0.0, 7.5]])
    assert tj.greedy_gap(lg).tolist() == [0.0, 0.75, 7.5]
    # router gap at k: k-th minus (k+1)-th largest
    r = np.array([[0.1, 0.9, 0.5, 0.7], [2.0, 2.0, 1.0, -1.0]])
    assert np.allclose(tj.router_gap(r, 1), [0.2, 0.0])
    assert np.allclose(tj.router_gap(r, 2), [0.2, 1.0])
    assert np.allclose(tj.router_gap(r, 3), [0.4, 2.0])
    # k = E: nothing is left out, so no decision can flip
    assert np.all(np.isinf(tj.router_gap(r, 4)))


def test_run_minimum_gaps():
    run = tj.Run()
    tr = od.StepTrace()
    tr.router_logits = [np.array([[0.3, 0.1, 0.2]]), np.array([[1.0, 0.95, 0.0]])]
    run.traces.append(tr)
    run.logits = [np.array([[1.0, 0.5]]), np.array([[2.0, 1.9, 0.0]])]
    assert math.isclose(run.min_router_gap(1), 0.05)
    assert math.isclose(run.min_router_gap(2), 0.1)
    assert math.isclose(run.min_greedy_gap(), 0.1)


# ------------------------------------------------------------ FP8 weights ----
# R19 / R20: OCP E4M3 codes with per-hidden-unit scales (the roadmap's FP8
# weights, megakernel post, Chinese version, section "下一步").

def test_e4m3_every_code_matches_the_library_decode():
    """All 256 codes against torch's float8_e4m3fn conversion (a library
    routine of the same OCP format); NaN codes are NaN on both sides."""
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = od.e4m3_to_float(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.isnan(got).sum() == 2                     # 0x7F and 0xFF only
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))


def test_e4m3_closed_form_values():
    """Values fixed by the format's definition: bias 7, 3 mantissa bits,
    subnormals m * 2^-9, largest finite 448, sign in the top bit."""
    cases = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0, 0x39: 1.125,
             0x3C: 1.5, 0x40: 2.0, 0x77: 240.0, 0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0, 0x81: -(2.0 ** -9)}
    for c, v in cases.items():
        assert od.e4m3_to_float(np.array([c], dtype=np.uint8))[0] == v, hex(c)
    assert np.signbit(od.e4m3_to_float(np.array([0x80], dtype=np.uint8))[0])


def test_fp8_scales_run_along_the_hidden_unit():
    """Gate and up scales multiply columns (hidden unit f of [H, F]); down
    scales multiply rows (hidden unit f of [F, H]): with every code 1.0 each
    weight equals its unit's scale, and distinct scales expose a transposed
    or swapped scale vector."""
    H, F = 3, 4
    one = np.full((H, F), 0x38, dtype=np.uint8)
    sg = np.array([1.0, 2.0, 4.0, 8.0], dtype=np.float32)
    su, sd = sg * 3, sg * 5
    wg, wu, wd = od.fp8_ffn_weights(one, one, one.T.copy(), sg, su, sd)
    assert np.array_equal(wg, np.tile(sg.astype(np.float64), (H, 1)))
    assert np.array_equal(wu, np.tile(su.astype(np.float64), (H, 1)))
    assert np.array_equal(wd, np.tile(sd.astype(np.float64)[:, None], (1, H)))


def test_fp8_dequantization_inverts_the_input_quantizer():
    """The oracle's decode of codes made by the input generator's quantizer
    (torch's cast) reproduces each weight within half a step of E4M3 at its
    magnitude: 2^-4 relative in the normal range, 2^-10 * scale below it."""
    g = torch.Generator().manual_seed(5)
    wg = (torch.randn(2, 64, 48, generator=g) * 0.02).to(torch.bfloat16)
    wu = (torch.randn(2, 64, 48, generator=g) * 0.02).to(torch.bfloat16)
    wd = (torch.randn(2, 48, 64, generator=g) * 0.02).to(torch.bfloat16)
    cg, cu, cd, sg, su, sd = (t.numpy() for t in gen.quantize_ffn_fp8(wg, wu, wd))
    for e in range(2):
        dq = od.fp8_ffn_weights(cg[e], cu[e], cd[e], sg[e], su[e], sd[e])
        for w, d, s in zip((wg[e], wu[e], wd[e]), dq, (sg[e][None, :], su[e][None, :], sd[e][:, None])):
            w = w.double().numpy()
            s = s.astype(np.float64)
            normal = np.abs(w) / s >= 2.0 ** -6
            err = np.abs(d - w)
            assert np.all(err[normal] <= 2.0 ** -4 * np.abs(w[normal]) * (1 + 1e-6))
            assert np.all(err[~normal] <= (2.0 ** -10 * np.broadcast_to(s, w.shape))[~normal] * (1 + 1e-6))
            # the largest magnitude of each vector is exactly code 448
            assert np.allclose(np.abs(d).max(axis=0 if s.shape[0] == 1 else 1), 448.0 * s.ravel(), rtol=1e-12)


class _Fp8View:
    """bf16 weights W with FP8 codes and scales for the FFNs (test input)."""

    def __init__(self, W, q):
        self.W, self.q = W, q

    def __call__(self, *a):
        return self.W(*a)

    def fp8_ffn(self, l, e):
        return self.q[(l, e)]


@pytest.mark.parametrize("dense", [False, True])
def test_decode_step_with_fp8_weights_equals_the_same_values_in_bf16(dense):
    """FP8 codes times power-of-two scales are exact bf16 values: a step with
    those FFN weights given as codes and scales equals, bit for bit, the step
    with the same values given as bf16 weights (the FP8 path feeds the gate,
    up and down matrices to the same places)."""
    cfg = configs.small_variant(configs.TINY_DENSE if dense else configs.TINY, n_layers=2)
    w = gen.make_weights(cfg, seed=3, device="cpu")
    rng = np.random.default_rng(4)
    E = 1 if dense else cfg.n_experts
    H, F = cfg.hidden, cfg.expert_ffn
    q = {}
    for l in range(cfg.n_layers):
        bf = {}
        for k, shape in (("wg", (E, H, F)), ("wu", (E, H, F)), ("wd", (E, F, H))):
            # codes of magnitude 2^-6 .. 448 with random signs, scales 2^-12 .. 2^-9
            codes = rng.integers(0x08, 0x7F, size=shape).astype(np.uint8) | (rng.integers(0, 2, shape) << 7).astype(np.uint8)
            scales = np.exp2(rng.integers(-12, -8, size=(E, F))).astype(np.float32)
            bf[k] = (codes, scales)
            vals = od.e4m3_to_float(codes) * (scales[:, None, :] if k != "wd" else scales[:, :, None])
            w[f"{k}.{l}"] = torch.from_numpy(vals).to(torch.bfloat16)
            assert np.array_equal(w[f"{k}.{l}"].double().numpy(), vals)
        for e in range(E):
            q[(l, e)] = (bf["wg"][0][e], bf["wu"][0][e], bf["wd"][0][e], bf["wg"][1][e], bf["wu"][1][e], bf["wd"][1][e])
    W = gen.NumpyWeights(w)
    V = _Fp8View(W, q)
    toks = np.array([5, 77]) if not dense else np.array([9, 31])
    bt = np.array([[0], [1]])
    lens = np.array([1, 1])
    a, _ = od.decode_step(cfg, W, _empty_pool(cfg, 2), bt, toks, lens, dtype=np.float64)
    b, _ = od.decode_step(cfg, V, _empty_pool(cfg, 2), bt, toks, lens, dtype=np.float64)
    assert np.array_equal(a, b)
    # and a swapped gate/up pair would not be equal
    q2 = {k: (v[1], v[0]) + v[2:] for k, v in q.items()}
    c, _ = od.decode_step(cfg, _Fp8View(W, q2), _empty_pool(cfg, 2), bt, toks, lens, dtype=np.float64)
    assert not np.array_equal(a, c)
