#!/usr/bin/env python3
"""Decode throughput of the persistent decode megakernel on one MI355X.

Workload: the 48-layer parallel-transformer MoE model (hidden 2048, 32 query /
4 kv heads of 128, 128 experts top-8 of width 768, vocab 131072, 12 full and
36 sliding-window-4096 layers) with random bf16 weights, batch 1, an 8K
context of synthetic N(0,1) bf16 KV; greedy decoding, the kernel feeding each
step's token and length to the next (MK_STEP_ADVANCE). A step is one decode
step of the whole model (one megakernel launch). Inputs are resident in HBM
before the timed region; the timed region is bracketed by stream syncs and
HIP events on the stream the kernel runs on.

Also reported on the same inputs: the kernel-per-op variant's rate (A/B), the
algorithmic-bytes roofline of the megakernel, and the oracle's rate on the
host cores for one step (a baseline, not a target).

Prints one JSON line. One GPU only: --gpus above 1 exits with a message.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="full48_b1_8k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ab", action="store_true", help="skip the kernel-per-op comparison")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "megakernel_traffic.json"),
                    help="HBM bytes per launch measured by rocprofv3 counters (if present)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the decode step "
              "runs on a single MI355X, with no collectives)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import moe_persistent_decode_amd as mk
    from moe_persistent_decode_amd import sol
    from mkinputs import configs, gen

    wl = configs.WORKLOADS[args.workload]
    m = wl.model
    B = wl.batch
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    W, K = args.warmup, args.steps
    runs = 2 if not args.no_ab else 1
    extra = runs * (W + K) + 1
    bs = gen.make_batch(wl, extra_steps=extra)
    max_seq = int(bs.seq_lens.max()) + extra
    log(f"[bench] {wl.name}: B={B} seq_len={wl.seq_len} pages={bs.n_pages} steps={K} warmup={W}")

    t0 = time.time()
    pool = gen.make_kv_pool(m, bs.n_pages, seed=wl.seed_kv, device=dev)
    pool_host0 = gen.bf16_bits(pool) if not args.no_cpu_baseline else None
    cfg = mk.make_config(m, B, max_seq, bs.n_pages, bs.max_pages_per_seq, mk.MODE_MEGAKERNEL)
    dec = mk.Decoder(cfg, pool)
    g = {n: gen.weight_tensor(m, n, wl.seed_weights, dev) for n in gen.GLOBAL_NAMES}
    dec.load_globals(g["emb"], g["gamma_f"], g["wlm"])
    del g
    for l in range(m.n_layers):
        w = gen.make_layer_weights(m, l, wl.seed_weights, dev)
        dec.load_layer(l, *(w[f"{k}.{l}"] for k in gen.LAYER_KINDS))
        stream.synchronize()
        del w
    torch.cuda.synchronize()
    log(f"[bench] inputs drawn and loaded in {time.time() - t0:.1f}s")

    tokens = bs.tokens.to(dev)
    seq_lens = bs.seq_lens.to(dev)
    bt = bs.block_tables.to(dev)
    logits = torch.empty((B, m.vocab), dtype=torch.float32, device=dev)
    seq0 = int(bs.seq_lens.max())
    state = {"seq": seq0}

    def run(n):
        for _ in range(n):
            dec.step(tokens, bt, seq_lens, state["seq"], logits, advance=True, stream=stream)
            state["seq"] += 1

    def timed(mode):
        dec.set_mode(mode)
        run(W)
        dec.sync(stream)
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        seq_first = state["seq"]
        torch.cuda.synchronize()
        start.record(stream)
        run(K)
        end.record(stream)
        torch.cuda.synchronize()
        dec.sync(stream)
        ms = start.elapsed_time(end)
        return ms, seq_first

    ms_mk, seq_first = timed(mk.MODE_MEGAKERNEL)
    step_ms = ms_mk / K
    tok_s = B * K / (ms_mk / 1e3)
    # algorithmic bytes per step, averaged over the timed steps (batch 1: k distinct experts)
    n_active = [min(m.top_k * B, m.n_experts)] * m.n_layers
    bytes_avg = float(np.mean([sol.step_bytes(m, [seq_first + i] * B, n_active) for i in range(K)]))
    achieved = bytes_avg / (step_ms / 1e3) / 1e9
    log(f"[bench] megakernel: {step_ms:.3f} ms/step, {tok_s:.1f} tok/s, {achieved:.0f} GB/s "
        f"({achieved / 8000:.1%} of 8 TB/s)")

    traffic = None
    if os.path.exists(args.traffic_json):
        try:
            tj = json.load(open(args.traffic_json))
            if tj.get("workload") == wl.name:
                traffic = tj.get("hbm_bytes_per_launch")
        except Exception:
            traffic = None

    out = {
        "metric": "decode tok/s at batch 1 and 32, 8K ctx; HBM GB/s as % of MI355X peak",
        "value": round(tok_s, 2),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": B, "seq_len": seq0, "decode": "greedy, in-kernel advance"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": 8000.0, "unit": "GB/s",
                     "frac": round(achieved / 8000.0, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": int(bytes_avg), "kernel": "mk_interp<128> (one launch per step)"},
    }

    if not args.no_ab:
        ms_op, _ = timed(mk.MODE_KERNEL_PER_OP)
        out["kernel_per_op"] = {"ms_per_step": round(ms_op / K, 4), "tok_s": round(B * K / (ms_op / 1e3), 2),
                                "megakernel_speedup": round(ms_op / ms_mk, 3)}
        log(f"[bench] kernel-per-op: {ms_op / K:.3f} ms/step -> megakernel {ms_op / ms_mk:.2f}x")
        dec.set_mode(mk.MODE_MEGAKERNEL)

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(m, wl, bs, pool_host0)
        log(f"[bench] oracle on host: {out['cpu_baseline']}")

    dec.close()
    print(json.dumps(out), flush=True)


def cpu_baseline(m, wl, bs, pool_host0):
    """The oracle (test infrastructure) timed on the host for one decode step of
    the same workload: weights drawn lazily on the GPU and kept in host memory
    by a first, untimed run; the second run is timed."""
    import numpy as np

    from mkinputs import gen
    from oracle import decode as od

    W = gen.LazyWeights(m, wl.seed_weights, device="cuda")
    bt = bs.block_tables.numpy()
    toks = bs.tokens.numpy()
    lens = bs.seq_lens.numpy()
    pool = pool_host0.copy()
    od.decode_step(m, W, pool, bt, toks, lens)
    t = time.time()
    od.decode_step(m, W, pool, bt, toks, lens)
    dt = time.time() - t
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count()
    return {"value": round(wl.batch / dt, 4), "unit": "tok/s", "cores": cores, "kind": "oracle",
            "sample": f"1 decode step of {wl.name} (batch {wl.batch}, seq_len {int(lens.max())}), "
                      f"weights resident in host memory; {dt:.1f} s"}


if __name__ == "__main__":
    main()
