"""CPU tests of the C ABI: exports, host-side validation, the task schedule.

No GPU is touched: the library is loaded, every function that include/mk.h
declares must be exported, and host-only handles (mk_create_host_only) build
and simulate the per-CU task lists of the persistent kernel.
"""
import ctypes
import os
import re

import numpy as np
import pytest

from mkinputs import configs
from moe_persistent_decode_amd import sol

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    text = open(os.path.join(ROOT, "include", "mk.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(mk_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_function():
    import moe_persistent_decode_amd as mk
    declared = _header_functions()
    assert len(declared) >= 15, declared
    lib = ctypes.CDLL(mk.LIB_PATH)
    missing = [f for f in declared if not hasattr(lib, f)]
    assert not missing, missing
    assert sorted(mk.EXPORTS) == declared


def _host(m, batch=1, max_seq=8192 + 64, n_cus=256, mode=0):
    import moe_persistent_decode_amd as mk
    from moe_persistent_decode_amd.binding import Decoder
    P = m.page_size
    mpps = -(-max_seq // P)
    cfg = mk.make_config(m, batch, max_seq, mpps * batch, mpps, mode)
    return Decoder(cfg, host_only_cus=n_cus)


def _bad(m, **kw):
    import moe_persistent_decode_amd as mk
    from moe_persistent_decode_amd.binding import Decoder
    cfg = mk.make_config(m, 1, 1024, 64, 64, 0)
    for k, v in kw.items():
        setattr(cfg, k, v)
    with pytest.raises(mk.MkError) as e:
        Decoder(cfg, host_only_cus=256)
    return e.value


@pytest.mark.parametrize("field,value", [
    ("hidden", 300), ("hidden", 4096), ("head_dim", 96), ("n_q_heads", 5), ("n_q_heads", 64), ("n_experts", 12),
    ("top_k", 9), ("top_k", 0), ("expert_ffn", 100), ("vocab", 1000), ("page_size", 32),
    ("n_layers", 0), ("max_batch", 0), ("max_batch", 33), ("n_pages", 0), ("rms_eps", -1.0),
])
def test_invalid_configs_are_rejected(field, value):
    err = _bad(configs.TINY, **{field: value})
    assert err.status in (1, 2), err


def test_schedule_full_model_batch1():
    m = configs.FULL48
    d = _host(m)
    info = d.schedule_info(1, 8192)
    assert info.n_cus == 256
    # round-robin placement, except the O projections, which go to the compute
    # units that ran the layer's attention (fewer than all in window layers)
    assert info.max_tasks_per_cu <= 2 * -(-info.n_tasks // 256)
    tasks, off = d.schedule_export(1, 8192)
    assert off[0] == 0 and off[-1] == info.n_tasks and np.all(np.diff(off) >= 0)
    ops = tasks[:, 0] & 0xFF
    # every layer's QKV covers the projection's output panels exactly once
    assert np.count_nonzero(ops == 10) >= 1  # LM head tasks
    # weight bytes the schedule streams: all dense weights, the LM head and 8 experts per layer
    exp = sum(sol.layer_weight_bytes(m) - 2 * m.hidden for _ in range(m.n_layers))
    assert info.weight_bytes_per_step >= exp
    st, msg = d.simulate(1, 8192, [m.top_k] * m.n_layers, seed=1)
    assert st == 0, msg
    d.close()


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_schedule_simulation_random_routing_completes(seed):
    m = configs.small_variant(configs.FULL48, n_layers=4)
    d = _host(m)
    rng = np.random.default_rng(seed)
    st, msg = d.simulate(1, 8192, rng.integers(1, m.top_k + 1, size=m.n_layers), seed=seed)
    assert st == 0, msg
    d.close()


def test_schedule_simulation_detects_a_lost_signal():
    """Dropping one task's signal must leave a waiter unsatisfied (the
    simulator reports the deadlock rather than completing)."""
    m = configs.small_variant(configs.FULL48, n_layers=2)
    d = _host(m)
    info = d.schedule_info(1, 4096)
    st_ok, _ = d.simulate(1, 4096, [8, 8], seed=0)
    assert st_ok == 0
    st, msg = d.simulate(1, 4096, [8, 8], seed=0, corrupt_task=info.n_tasks // 3)
    assert st != 0 and msg
    d.close()


def test_schedule_tiny_model_on_few_cus():
    d = _host(configs.TINY, max_seq=256, n_cus=4)
    st, msg = d.simulate(1, 200, [2, 2], seed=3)
    assert st == 0, msg
    d.close()


# ---- speed-of-light arithmetic against the megakernel post's numbers
# (section "What is a Megakernel?" / introduction: a 30B model with 3.3B active
# parameters streams 6.6 GB of bf16 weights plus about 0.5 GB of KV at 8K per
# step; at 3.35 TB/s that is about 470 tok/s)

def test_model_sizes_match_the_posts_description():
    total, active = configs.FULL48.param_counts()
    assert abs(total / 1e9 - 30.4) < 0.5
    assert abs(active / 1e9 - 3.3) < 0.05
    kv = sum(min(8192, configs.FULL48.layer_window(l)) or 8192 for l in range(48)) \
        * sol.kv_bytes_per_token(configs.FULL48)
    assert abs(kv / 1e9 - 0.5) < 0.01


def test_sol_reproduces_the_posts_470_tok_s():
    m = configs.FULL48
    _, active = m.param_counts()
    kv = sum(min(8192, m.layer_window(l)) or 8192 for l in range(48)) * sol.kv_bytes_per_token(m)
    post_bytes = 2 * active + kv
    assert abs(sol.sol_tokens_per_s(post_bytes, 1, 3.35e12) - 470) < 10
    # step_bytes streams the same except the embedding table (one row is read)
    # and adds the token's K/V append and the fp32 logits written
    b = sol.step_bytes(m, [8192], [8] * 48)
    emb = 2 * m.vocab * m.hidden
    extra = 48 * sol.kv_bytes_per_token(m) + 2 * m.hidden + 4 * m.vocab
    assert b == post_bytes - emb + extra


def test_step_bytes_window_and_batch():
    m = configs.FULL48
    one = sol.step_bytes(m, [100], [8] * 48)
    two = sol.step_bytes(m, [100, 100], [8] * 48)
    per_seq = 48 * 101 * sol.kv_bytes_per_token(m) + 2 * m.hidden + 4 * m.vocab
    assert two - one == per_seq
    # beyond the window only full layers grow
    a = sol.step_bytes(m, [5000], [8] * 48)
    b = sol.step_bytes(m, [5001], [8] * 48)
    assert b - a == 12 * sol.kv_bytes_per_token(m)


@pytest.mark.parametrize("batch,seq", [(1, 8192), (4, 65536), (8, 16384)])
def test_fixed_moe_shares_follow_the_placement(batch, seq):
    """MoE claimers with fixed shares (fused up to 4 tokens): per layer the
    indices are a permutation of the claimers, those on compute units without
    an attention claimer in that layer come first, and their count is the one
    the tasks carry."""
    m = configs.FULL48 if batch == 1 else configs.small_variant(configs.FULL48, n_layers=2)
    d = _host(m, batch=batch, max_seq=seq + 64)
    tasks, off = d.schedule_export(batch, seq)
    ops, layer = tasks[:, 0] & 0xFF, tasks[:, 1]
    cu = np.searchsorted(off, np.arange(len(tasks)), side="right") - 1
    want_op = 9 if batch <= 4 else 8
    for l in range(m.n_layers):
        moe = np.nonzero((ops == want_op) & (layer == l))[0]
        assert len(moe) > 0
        attn_cus = set(cu[(ops == 3) & (layer == l)].tolist())
        k, nf, nt = tasks[moe, 16], tasks[moe, 17], tasks[moe, 18]
        assert np.all(nt == len(moe)) and sorted(k.tolist()) == list(range(len(moe)))
        free = np.array([c not in attn_cus for c in cu[moe]])
        assert np.all(nf == free.sum())
        assert np.all(k[free] < nf[0]) and np.all(k[~free] >= nf[0])
    d.close()


@pytest.mark.parametrize("batch", [1, 4])
def test_fused_moe_residual_tasks(batch):
    """Fused MoE layers: one residual task per column block, each waiting for
    every claimer and O projection of its layer (plain arrivals on one
    counter) and signalling the next layer's input; no task of the layer uses
    the per-block arrival counters."""
    m = configs.small_variant(configs.FULL48, n_layers=3)
    d = _host(m, batch=batch, max_seq=8192 + 64)
    tasks, off = d.schedule_export(batch, 8192)
    ops, layer = tasks[:, 0] & 0xFF, tasks[:, 1]
    wait_c, wait_t, sig = tasks[:, 8:11], tasks[:, 11:14], tasks[:, 14]
    NB = m.hidden // 64
    for l in range(m.n_layers):
        res = np.nonzero((ops == 4) & (layer == l))[0]
        assert sorted(tasks[res, 2].tolist()) == list(range(NB))
        moe = np.nonzero((ops == 9) & (layer == l))[0]
        op = np.nonzero((ops == 5) & (layer == l))[0]
        fin = set(sig[moe].tolist()) | set(tasks[op, 4].tolist())
        assert len(fin) == 1 and np.all(tasks[op, 16] == 1)
        (fin,) = fin
        for r in res:
            j = list(wait_c[r]).index(fin)
            assert wait_t[r, j] == len(moe) + len(op)
        assert len(set(sig[res].tolist())) == 1
    d.close()


def test_host_only_handle_has_no_kv_pool_and_takes_a_wait_limit():
    import moe_persistent_decode_amd as mk
    d = _host(configs.TINY)
    with pytest.raises(mk.MkError) as e:
        d.kv_cache(0)
    assert e.value.status == 7  # MK_ERR_STATE
    d.set_wait_limit(50)        # stored for later steps
    d.set_wait_limit(0)         # back to the default
    d.close()


@pytest.mark.parametrize("order", [0, 1, 2])
@pytest.mark.parametrize("placement", [0, 1, 2])
@pytest.mark.parametrize("batch", [1, 2, 4, 8, 17, 32])
def test_schedule_options_simulate_without_deadlock(order, placement, batch):
    """Every wave order and placement (the scheduler ablation) gives per-CU
    lists that run to completion on the host model, with every counter at the
    count of arrivals it expects, under random routing outcomes: the fused MoE
    (at most 4 tokens), fixed shares (at most 16) and claiming (above)."""
    m = configs.small_variant(configs.FULL48, n_layers=4)
    d = _host(m, batch=batch, max_seq=16384 + 64)
    d.set_schedule_options(order, placement)
    rng = np.random.default_rng(order * 100 + placement * 10 + batch)
    hi = min(m.n_experts, batch * m.top_k)
    for seed in range(2):
        n_active = rng.integers(max(m.top_k, hi // 2), hi + 1, size=m.n_layers)
        st, msg = d.simulate(batch, 16384 if batch > 4 else 8192, n_active, seed=seed)
        assert st == 0, (msg, n_active)
    d.close()


def test_schedule_options_change_the_lists():
    m = configs.small_variant(configs.FULL48, n_layers=4)
    d = _host(m, batch=1)
    seen = set()
    for order in range(3):
        for placement in range(3):
            d.set_schedule_options(order, placement)
            t, off = d.schedule_export(1, 8192)
            seen.add(hash(t.tobytes() + off.tobytes()))
    # (attention-first moves the O projections only within their own units
    # under the tuned placements: some pairs coincide)
    assert len(seen) >= 6
    import moe_persistent_decode_amd as mk
    with pytest.raises(mk.MkError):
        d.set_schedule_options(3, 0)
    with pytest.raises(mk.MkError):
        d.set_schedule_options(0, 5)
    d.close()


def test_decode_service_needs_a_device_handle():
    import moe_persistent_decode_amd as mk
    d = _host(configs.TINY)
    with pytest.raises(mk.MkError) as e:
        mk.DecodeService(d, max_batch=1, page0=0, n_pages=8)
    assert e.value.status == 7  # MK_ERR_STATE
    d.close()


@pytest.mark.parametrize("batch,ctx", [(1, 8192), (1, 262144), (4, 65536), (2, 131072), (32, 16384)])
def test_attention_splits_cover_the_keys_and_spread_at_long_context(batch, ctx):
    """The attention splits of every layer cover its keys (a window layer's
    window, a full layer's whole context, one page of slack for a window that
    straddles pages), stay within the combine's 256, and at long contexts
    spread a full layer's keys over one to about two items per compute unit
    (256 units) -- the schedule then simulates to completion."""
    m = configs.small_variant(configs.FULL48, n_layers=4)
    d = _host(m, batch=batch, max_seq=ctx + 64)
    t, _ = d.schedule_export(batch, ctx)
    attn = t[t[:, 0] == 3]
    for layer in range(m.n_layers):
        a = attn[attn[:, 1] == layer]
        ns, pps = int(a[0, 5]), int(a[0, 6])
        assert (a[:, 5] == ns).all() and (a[:, 6] == pps).all()
        keys = min(ctx, m.layer_window(layer) or ctx)
        pages = -(-keys // m.page_size) + 1
        assert ns * pps >= pages and (ns - 1) * pps < pages and ns <= 256, (layer, ns, pps, pages)
        if not m.layer_window(layer) and ctx >= 65536:
            assert 256 <= batch * m.n_kv_heads * ns <= 640, (layer, ns, pps)
    hi = min(m.n_experts, batch * m.top_k)
    st, msg = d.simulate(batch, ctx, [hi] * m.n_layers, seed=batch)
    assert st == 0, msg
    d.close()


def test_stream_read_rejects_bad_buffers_on_the_host():
    """mk_stream_read checks alignment and size before any device call."""
    from moe_persistent_decode_amd.binding import lib
    assert lib.mk_stream_read(ctypes.c_void_p(4096), 0, None) == 1
    assert lib.mk_stream_read(ctypes.c_void_p(4099), 64, None) == 1
    assert lib.mk_stream_read(ctypes.c_void_p(4096), 40, None) == 1
    assert lib.mk_stream_read(None, 64, None) == 1


@pytest.mark.parametrize("model", ["tiny_dense", "llama1b"])
@pytest.mark.parametrize("batch", [1, 2, 4])
def test_dense_schedule_simulates(model, batch):
    """A dense model's per-CU lists (QKV, attention, O projection, the mid
    residual, the FFN over every unit, the final residual) run to completion
    on the host model with every counter at its expected count; no router."""
    m = configs.TINY_DENSE if model == "tiny_dense" else configs.LLAMA1B
    d = _host(m, batch=batch, max_seq=8192 + 64)
    t, off = d.schedule_export(batch, 8192)
    ops = np.bincount(t[:, 0], minlength=11)
    assert ops[6] == 0 and ops[8] == 0                       # no router, no claiming MoE
    assert ops[9] == 256 * m.n_layers                         # one FFN claimer per unit and layer
    assert ops[4] == 2 * (m.hidden // (64 if m.hidden >= 1024 else 32)) * m.n_layers  # two residuals per block
    res = t[t[:, 0] == 4]
    assert sorted(set(res[:, 3].tolist())) == [1, 2]          # mid and final residual modes
    for seed in range(2):
        st, msg = d.simulate(batch, 8192, [1] * m.n_layers, seed=seed)
        assert st == 0, msg
    d.close()


def test_dense_config_limits():
    import moe_persistent_decode_amd as mk
    from moe_persistent_decode_amd.binding import Decoder, MkError
    m = configs.TINY_DENSE
    for kw, bad in ((dict(max_batch=5), "at most"), (dict(n_experts=2), "n_experts"),
                    (dict(expert_ffn=8320), "FFN width")):
        cfg = mk.make_config(m, kw.get("max_batch", 1), 1024, 64, 64, 0)
        for k, v in kw.items():
            setattr(cfg, k, v)
        with pytest.raises(MkError, match=bad):
            Decoder(cfg, host_only_cus=256)


@pytest.mark.parametrize("model,batch", [("full48", 1), ("full48", 4), ("full48", 8), ("full48", 32),
                                         ("llama1b", 1), ("llama1b", 4)])
def test_cost_model_and_random_placements_simulate(model, batch):
    """The greedy cost-model placement and seeded random candidates (the
    post's two other schedulers) keep every list in flat order with a wave's
    claimers on distinct units: they run to completion on the host model, and
    candidates differ by seed."""
    import moe_persistent_decode_amd as mk
    m = configs.small_variant(configs.FULL48, n_layers=4) if model == "full48" else \
        configs.small_variant(configs.LLAMA1B, n_layers=4)
    d = _host(m, batch=batch, max_seq=16384 + 64)
    seq = 16384 if batch > 4 else 8192
    hi = 1 if m.dense else min(m.n_experts, batch * m.top_k)
    seen = set()
    for placement, seeds in ((mk.PLACE_COST_MODEL, [1]), (mk.PLACE_RANDOM, [1, 2, 3])):
        d.set_schedule_options(0, placement)
        for sd in seeds:
            d.set_placement_seed(sd)
            t, off = d.schedule_export(batch, seq)
            seen.add(hash(t.tobytes() + off.tobytes()))
            # a wave's claimers on distinct units: at most one claimer task
            # per (unit, layer, opcode)
            for cu in range(len(off) - 1):
                lst = t[off[cu]:off[cu + 1]]
                cl = lst[np.isin(lst[:, 0], [3, 8, 9])]
                keys = set()
                for row in cl:
                    assert (int(row[0]), int(row[1])) not in keys, (placement, sd, cu)
                    keys.add((int(row[0]), int(row[1])))
            st, msg = d.simulate(batch, seq, [hi] * m.n_layers, seed=sd)
            assert st == 0, (placement, sd, msg)
    assert len(seen) == 4
    d.close()


def _hz_models():
    return {"full48": configs.small_variant(configs.FULL48, n_layers=4), "tiny_win": configs.TINY_WIN,
            "llama1b": configs.small_variant(configs.LLAMA1B, n_layers=4)}


@pytest.mark.parametrize("model", ["full48", "tiny_win", "llama1b"])
@pytest.mark.parametrize("batch", [1, 2, 4, 8, 17, 32])
def test_no_read_before_arrive_in_any_schedule(model, batch):
    """The per-buffer tag check (mk_schedule_check) finds no read before its
    writer is known to have finished and no overwrite before a reader is, for
    every wave order and placement (tuned, round-robin, affinity, cost model,
    three random candidates)."""
    import moe_persistent_decode_amd as mk
    m = _hz_models()[model]
    if m.dense and batch > 4:
        pytest.skip("dense models decode at most 4 sequences")
    d = _host(m, batch=batch, max_seq=16384 + 64)
    seq = 16384 if batch > 4 else 8192
    for order in range(3):
        for placement, seeds in ((0, [1]), (1, [1]), (2, [1]), (mk.PLACE_COST_MODEL, [1]), (mk.PLACE_RANDOM, [3, 7, 9])):
            d.set_schedule_options(order, placement)
            for sd in seeds:
                d.set_placement_seed(sd)
                st, rep = d.check_hazards(batch, seq)
                assert st == 0, (order, placement, sd, rep)
    d.close()


def test_hazard_check_finds_the_early_residual_stream_read():
    """The residual task of an earlier version loaded its block of the
    residual stream before any wait. Modelled that way, the check reports it
    for the random placement under which the GPU gave wrong logits (batch 4,
    seed 7) and not for the tuned placement, where every unit runs a task that
    waited for the layer's input before its residual task."""
    import moe_persistent_decode_amd as mk
    d = _host(configs.TINY_WIN, batch=4, max_seq=8192 + 64)
    st, rep = d.check_hazards(4, 8192, flags=1)
    assert st == 0, rep
    d.set_schedule_options(0, mk.PLACE_RANDOM)
    d.set_placement_seed(7)
    st, rep = d.check_hazards(4, 8192, flags=1)
    assert st != 0 and "read before its writer" in rep and " on h[" in rep, rep
    st, rep = d.check_hazards(4, 8192)
    assert st == 0, rep
    d.close()


@pytest.mark.parametrize("model", ["full48", "llama1b"])
def test_hazard_check_finds_a_planted_missing_wait(model):
    m = _hz_models()[model]
    d = _host(m, batch=1, max_seq=8192 + 64)
    st, rep = d.check_hazards(1, 8192, flags=2)
    assert st != 0 and "read before its writer" in rep, rep
    d.close()


@pytest.mark.parametrize("name,batch,ctx", [("full48", 1, 8192), ("full48", 32, 16384), ("full48", 1, 262144),
                                            ("full48", 4, 65536), ("llama1b", 1, 8192), ("llama1b", 4, 16384)])
def test_no_read_before_arrive_at_full_size(name, batch, ctx):
    """The benchmark schedules themselves (48 or 16 layers, shipped order,
    tuned placement) pass the per-buffer tag check."""
    m = configs.FULL48 if name == "full48" else configs.LLAMA1B
    d = _host(m, batch=batch, max_seq=ctx + 64)
    st, rep = d.check_hazards(batch, ctx)
    assert st == 0, rep
    d.close()


def test_litmus_rejects_bad_arguments_on_the_host():
    """mk_litmus_message_passing checks its sizes and mode before any device
    call: pairs in [1, 512], rounds in [1, 1e6], coherent in [0, 2]."""
    from moe_persistent_decode_amd.binding import lib
    s, t = ctypes.c_uint32(0), ctypes.c_uint32(0)
    for pairs, rounds, mode in [(0, 10, 1), (513, 10, 1), (4, 0, 1), (4, 10, 3), (4, 10, -1)]:
        assert lib.mk_litmus_message_passing(0, pairs, rounds, mode, ctypes.byref(s), ctypes.byref(t)) == 1


def test_fp8_ffn_config_limits_and_loader_checks():
    """FP8 feed-forward weights: a 0/1 flag (a dense model keeps its batch
    limit of 4); a host-only handle takes no weights, and a bf16 handle
    refuses the FP8 loader. An FP8 handle's schedules simulate at every batch
    (the claiming MoE above 4 sequences)."""
    import moe_persistent_decode_amd as mk
    from moe_persistent_decode_amd.binding import Decoder, MkError
    cfg = mk.make_config(configs.TINY_DENSE, 5, 1024, 64, 64, 0, ffn_fp8=True)
    with pytest.raises(MkError, match="at most"):
        Decoder(cfg, host_only_cus=256)
    for m in (configs.TINY, configs.TINY_DENSE):
        cfg = mk.make_config(m, 4, 1024, 64, 64, 0)
        cfg.ffn_fp8 = 2
        with pytest.raises(MkError, match="ffn_fp8"):
            Decoder(cfg, host_only_cus=256)
    cfg = mk.make_config(configs.TINY, 4, 1024, 64, 64, 0, ffn_fp8=True)
    d = Decoder(cfg, host_only_cus=256)
    with pytest.raises(MkError, match="host-only"):
        d.load_ffn_fp8(0, 16, 16, 16, 16, 16, 16, stream=0)
    st, msg = d.simulate(4, 1000, [1] * configs.TINY.n_layers, seed=3)
    assert st == 0, msg
    d.close()
    for B in (5, 8, 16, 17, 32):
        cfg = mk.make_config(configs.FULL48, B, 8192 + 64, 520 * B, 520, 0, ffn_fp8=True)
        d = Decoder(cfg, host_only_cus=256)
        for seed in (1, 2):
            st, msg = d.simulate(B, 8192, [min(128, 8 * B)] * configs.FULL48.n_layers, seed=seed)
            assert st == 0, (B, msg)
        d.close()
    bf = _host(configs.TINY, batch=4, max_seq=1024)
    with pytest.raises(MkError, match="host-only|not an FP8"):
        bf.load_ffn_fp8(0, 16, 16, 16, 16, 16, 16, stream=0)
    bf.close()


@pytest.mark.parametrize("batch", [1, 4, 8, 16, 32])
def test_fp8_schedules_pass_the_hazard_check(batch):
    """An FP8 model's schedules (the claiming MoE from 5 sequences on, with
    the O projection as the claimers' item queue) pass the per-buffer tag
    check in every wave order and the tuned and round-robin placements."""
    import moe_persistent_decode_amd as mk
    from moe_persistent_decode_amd.binding import Decoder
    m = configs.FULL48
    mpps = -(-(16384 + 64) // m.page_size)
    d = Decoder(mk.make_config(m, batch, 16384 + 64, mpps * batch, mpps, 0, ffn_fp8=True), host_only_cus=256)
    for order in range(3):
        for placement in (0, 1):
            d.set_schedule_options(order, placement)
            st, rep = d.check_hazards(batch, 16384 if batch > 4 else 8192)
            assert st == 0, (order, placement, rep)
    d.close()
