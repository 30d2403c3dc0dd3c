"""GPU parity on the tiny 2-layer model (the HIP path through the C ABI vs the oracle).

Case: the recorded seed's weights, a 128-token context of uniform random
tokens whose KV the oracle builds, then 16 greedy steps. Every step's logits
must be within 3e-2 (max abs) and 1e-2 (relative L2) of the oracle's, every
greedy token and every layer's top-k expert set identical, and the appended
K/V within the bf16 operand rounding of the oracle's.
"""
import numpy as np
import pytest
import torch

from mkinputs import gen
from oracle import decode as od
from oracle import trajectory as tj
from tests.harness import bits_to_torch, logits_close, make_decoder, say, tiny_case, torch_to_bits

pytestmark = pytest.mark.gpu

MODES = [(0, "megakernel"), (1, "kernel_per_op")]


@pytest.fixture(scope="module")
def case():
    tc = tiny_case()
    cfg = tc.cfg
    pool = np.zeros(gen.kv_pool_shape(cfg, tc.bs.n_pages), np.uint16)
    ctx_run = tj.teacher_forced(cfg, tc.W, pool, tc.bs.block_tables.numpy(), tc.ctx, np.array([1]))
    return tc, pool, ctx_run


def _gpu_weights(tc):
    return {k: v.cuda() for k, v in tc.weights.items()}


def _check_kv(gpu_pool: np.ndarray, ref_pool: np.ndarray):
    """The appended K/V are bf16 roundings of projections whose operands the
    GPU rounds to bf16 (the layer input; from layer 1 on also the attention
    output), about 2e-3 relative each: every layer's cache must be within 1%
    of its largest value element-wise and 0.5% in relative L2 (a wrong slot,
    page, head or rotation is off by the values' own size)."""
    a = od.bf16_to_float(gpu_pool, np.float64)
    b = od.bf16_to_float(ref_pool, np.float64)
    d = np.abs(a - b)
    for l in range(a.shape[0]):
        scale = np.abs(b[l]).max()
        ulp = 2.0 ** (np.floor(np.log2(max(scale, 1e-30))) - 7)
        assert d[l].max() <= 1e-2 * scale + ulp, (l, float(d[l].max()), scale)
        assert np.linalg.norm(d[l]) <= 5e-3 * np.linalg.norm(b[l]) + ulp, (l, float(np.linalg.norm(d[l])))


@pytest.mark.parametrize("mode,name", MODES)
def test_tiny_greedy_decode_matches_oracle(case, mode, name):
    tc, ctx_pool, ctx_run = case
    cfg, wl = tc.cfg, tc.wl
    say(f"[tiny greedy {name}] seed={tc.W and 'rec'} steps={wl.steps}")
    pool_ref = ctx_pool.copy()
    bt = tc.bs.block_tables.numpy()
    g0 = ctx_run.greedy[-1]
    ref = tj.greedy_decode(cfg, tc.W, pool_ref, bt, g0, np.array([wl.seq_len[0]]), wl.steps)

    pool_gpu = bits_to_torch(ctx_pool)
    max_seq = wl.seq_len[0] + wl.steps
    dec = make_decoder(cfg, tc.bs, pool_gpu, max_seq, mode)
    dec.load_weights(_gpu_weights(tc))
    trace = torch.full((cfg.n_layers, 1, cfg.top_k), -1, dtype=torch.int32, device="cuda")
    dec.set_routing_trace(trace)
    tokens = torch.tensor(g0, dtype=torch.int32, device="cuda")
    seq_lens = torch.tensor([wl.seq_len[0]], dtype=torch.int32, device="cuda")
    bt_gpu = tc.bs.block_tables.cuda()
    logits = torch.empty((1, cfg.vocab), dtype=torch.float32, device="cuda")
    nxt = torch.empty(1, dtype=torch.int32, device="cuda")
    for s in range(wl.steps):
        dec.step(tokens, bt_gpu, seq_lens, int(seq_lens.item()), logits, nxt)
        dec.sync()
        lg = logits.cpu().numpy()
        ok, mx, rl2 = logits_close(lg[0], ref.logits[s][0])
        say(f"  step {s}: max|d|={mx:.2e} relL2={rl2:.2e} tok gpu={int(nxt.item())} ref={int(ref.greedy[s][0])}")
        assert ok, (s, mx, rl2)
        assert int(nxt.item()) == int(ref.greedy[s][0])
        tr = trace.cpu().numpy()
        for l in range(cfg.n_layers):
            assert sorted(tr[l, 0].tolist()) == sorted(ref.traces[s].topk_idx[l][0].tolist()), (s, l)
        tokens.copy_(nxt)
        seq_lens += 1
    _check_kv(torch_to_bits(pool_gpu), pool_ref)
    dec.close()


@pytest.mark.parametrize("mode,name", MODES)
def test_tiny_gpu_builds_context_itself(case, mode, name):
    """The GPU appends the whole context token by token (teacher-forced) from an
    empty cache; its logits at every step and the resulting cache match."""
    tc, ctx_pool, ctx_run = case
    cfg, wl = tc.cfg, tc.wl
    say(f"[tiny context {name}] {len(tc.ctx)} steps")
    pool_gpu = torch.zeros(gen.kv_pool_shape(cfg, tc.bs.n_pages), dtype=torch.bfloat16, device="cuda")
    dec = make_decoder(cfg, tc.bs, pool_gpu, wl.seq_len[0] + wl.steps, mode)
    dec.load_weights(_gpu_weights(tc))
    bt_gpu = tc.bs.block_tables.cuda()
    logits = torch.empty((1, cfg.vocab), dtype=torch.float32, device="cuda")
    worst = 0.0
    for t in range(len(tc.ctx)):
        tokens = torch.tensor(tc.ctx[t], dtype=torch.int32, device="cuda")
        seq_lens = torch.tensor([t + 1], dtype=torch.int32, device="cuda")
        dec.step(tokens, bt_gpu, seq_lens, t + 1, logits)
        dec.sync()
        ok, mx, rl2 = logits_close(logits.cpu().numpy()[0], ctx_run.logits[t][0])
        worst = max(worst, mx)
        assert ok, (t, mx, rl2)
    say(f"  worst max|d| over context: {worst:.2e}")
    _check_kv(torch_to_bits(pool_gpu), ctx_pool)
    dec.close()


def test_tiny_advance_flag_decodes_without_host(case):
    """MK_STEP_ADVANCE: the kernel writes the greedy token into tokens and bumps
    seq_lens, so back-to-back steps decode the same trajectory."""
    tc, ctx_pool, ctx_run = case
    cfg, wl = tc.cfg, tc.wl
    pool_ref = ctx_pool.copy()
    bt = tc.bs.block_tables.numpy()
    g0 = ctx_run.greedy[-1]
    ref = tj.greedy_decode(cfg, tc.W, pool_ref, bt, g0, np.array([wl.seq_len[0]]), wl.steps)
    pool_gpu = bits_to_torch(ctx_pool)
    dec = make_decoder(cfg, tc.bs, pool_gpu, wl.seq_len[0] + wl.steps, 0)
    dec.load_weights(_gpu_weights(tc))
    tokens = torch.tensor(g0, dtype=torch.int32, device="cuda")
    seq_lens = torch.tensor([wl.seq_len[0]], dtype=torch.int32, device="cuda")
    bt_gpu = tc.bs.block_tables.cuda()
    logits = torch.empty((1, cfg.vocab), dtype=torch.float32, device="cuda")
    toks = []
    for s in range(wl.steps - 1):
        dec.step(tokens, bt_gpu, seq_lens, wl.seq_len[0] + s + 1, logits, advance=True)
        toks.append(tokens.clone())
    dec.sync()
    got = [int(t.item()) for t in toks]
    assert got == [int(g[0]) for g in ref.greedy[:wl.steps - 1]]
    assert int(seq_lens.item()) == wl.seq_len[0] + wl.steps - 1
    dec.close()
