#!/usr/bin/env python3
"""Decode throughput of the persistent decode megakernel on one MI355X.

Workload (the line's `value`): the 48-layer parallel-transformer MoE model
(hidden 2048, 32 query / 4 kv heads of 128, 128 experts top-8 of width 768,
vocab 131072, 12 full and 36 sliding-window-4096 layers) with random bf16
weights, batch 1, an 8K context of synthetic N(0,1) bf16 KV; greedy decoding,
the kernel feeding each step's token and length to the next
(MK_STEP_ADVANCE). A step is one decode step of the whole model: one
megakernel launch. Inputs are resident in HBM before the timed region; the
timed region is bracketed by stream syncs and HIP events on the stream the
kernel runs on.

Also reported on the same line: the kernel-per-op variant's rate (A/B), the
algorithmic-bytes roofline of the megakernel (the distinct experts of every
step and layer counted from the kernel's own routing record), the same model
at batch 32 with ragged 512..16384 contexts over a shuffled page pool, and the
oracle's rate on the host cores (a baseline, not a target).

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

PEAK_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="full48_b1_8k")
    ap.add_argument("--batch-workload", default="full48_b32_ragged",
                    help="second measured workload, reported under second_workload ('none' to skip)")
    ap.add_argument("--long-workloads", default="full48_b1_256k,full48_b4_64k",
                    help="comma-separated long-context workloads timed after the others ('none' to skip)")
    ap.add_argument("--dense-workload", default="llama1b_b1_8k",
                    help="dense (Llama-3.2-1B-shaped) workload timed after the others ('none' to skip)")
    ap.add_argument("--fp8-workloads", default="full48_b1_8k,full48_b32_ragged,llama1b_b1_8k",
                    help="workloads measured again with FP8 feed-forward weights, reported under fp8_weights "
                         "('none' to skip)")
    ap.add_argument("--ffn-fp8", action="store_true",
                    help="measure the main workload with FP8 feed-forward weights (for profiling that path; the "
                         "headline line is the bf16 model's)")
    ap.add_argument("--fp8-op-trace", default=None, metavar="PATH",
                    help="write the per-opcode trace of the first FP8 workload's step (markdown)")
    ap.add_argument("--single-layer", default="layer1_b1_8k",
                    help="one-layer workload timed with the last-level cache flushed between steps ('none' to skip)")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the streaming-read ceiling diagnostic")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ab", action="store_true", help="skip the kernel-per-op comparison")
    ap.add_argument("--op-trace", default=None, metavar="PATH",
                    help="after timing, trace one more megakernel step per task and write a per-opcode summary (markdown)")
    ap.add_argument("--op-trace-raw", default=None, metavar="PATH",
                    help="with --op-trace: also save the raw per-task records (numpy .npy, int64 [tasks, 8])")
    ap.add_argument("--ablation", default=None, metavar="PATH",
                    help="instead of the benchmark line: time every wave order and placement of the scheduler "
                         "at batch 1, 2 and 4 (48 layers, 8K) and write the table (markdown) to PATH")
    ap.add_argument("--search", default=None, metavar="PATH",
                    help="time the cost-model and random placements against tuned and round-robin; write a table")
    ap.add_argument("--search-workloads", default="llama1b_b1_8k,full48_b1_8k")
    ap.add_argument("--search-candidates", type=int, default=200)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 256 MiB device-to-device copy (the reference for HBM byte counters)")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "megakernel_traffic.json"),
                    help="HBM bytes per launch measured by rocprofv3 counters (if present)")
    return ap.parse_args()


class Run:
    """One workload resident on the GPU: weights, KV pool, batch state."""

    def __init__(self, wl, steps, warmup, runs, fp8=False):
        import torch

        import moe_persistent_decode_amd as mk
        from mkinputs import gen
        self.wl, self.m, self.B, self.fp8 = wl, wl.model, wl.batch, fp8
        self.K, self.W = steps, warmup
        dev = torch.device("cuda:0")
        self.stream = torch.cuda.current_stream()
        extra = runs * (warmup + steps) + 2
        self.bs = gen.make_batch(wl, extra_steps=extra)
        self.max_seq = int(self.bs.seq_lens.max()) + extra
        t0 = time.time()
        self.pool = gen.make_kv_pool(self.m, self.bs.n_pages, seed=wl.seed_kv, device=dev)
        cfg = mk.make_config(self.m, self.B, self.max_seq, self.bs.n_pages, self.bs.max_pages_per_seq,
                             mk.MODE_MEGAKERNEL, ffn_fp8=fp8)
        self.dec = mk.Decoder(cfg, self.pool)
        g = {n: gen.weight_tensor(self.m, n, wl.seed_weights, dev) for n in gen.GLOBAL_NAMES}
        self.dec.load_globals(g["emb"], g["gamma_f"], g["wlm"])
        del g
        for l in range(self.m.n_layers):
            w = gen.make_layer_weights(self.m, l, wl.seed_weights, dev)
            if fp8:  # the drawn FFN weights as FP8 codes and scales
                self.dec.load_ffn_fp8(l, *gen.quantize_ffn_fp8(w.pop(f"wg.{l}"), w.pop(f"wu.{l}"), w.pop(f"wd.{l}")),
                                      stream=self.stream)
            self.dec.load_layer(l, *(w.get(f"{k}.{l}") for k in gen.layer_kinds(self.m)), stream=self.stream)
            self.stream.synchronize()
            del w
        torch.cuda.synchronize()
        log(f"[bench] {wl.name}{' (FP8 feed-forward weights)' if fp8 else ''}: B={self.B} lengths {int(self.bs.seq_lens.min())}..{int(self.bs.seq_lens.max())} "
            f"pages={self.bs.n_pages}; inputs drawn and loaded in {time.time() - t0:.1f}s")
        self.tokens = self.bs.tokens.to(dev)
        self.seq_lens = self.bs.seq_lens.to(dev)
        self.bt = self.bs.block_tables.to(dev)
        self.logits = torch.empty((self.B, self.m.vocab), dtype=torch.float32, device=dev)
        self.hint = int(self.bs.seq_lens.max())
        self.lens_host = self.bs.seq_lens.numpy().astype(int)
        self.done = 0  # steps decoded so far
        self.route = torch.full((steps, self.m.n_layers, self.B, self.m.top_k), -1, dtype=torch.int32, device=dev)

    def run(self, n, record=False, slot=0):
        for i in range(n):
            if record:
                self.dec.set_routing_trace(self.route[slot + i])
            self.dec.step(self.tokens, self.bt, self.seq_lens, self.hint + self.done, self.logits, advance=True,
                          stream=self.stream)
            self.done += 1
        if record:
            self.dec.set_routing_trace(None)

    def timed(self, mode, record=False):
        import torch
        self.dec.set_mode(mode)
        self.run(self.W)
        self.dec.sync(self.stream)
        first = self.done
        # an event after every step: the region's total and each step's time
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(self.K + 1)]
        torch.cuda.synchronize()
        ev[0].record(self.stream)
        for i in range(self.K):
            self.run(1, record, slot=i)
            ev[i + 1].record(self.stream)
        torch.cuda.synchronize()
        self.dec.sync(self.stream)
        self.step_ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(self.K)]
        return ev[0].elapsed_time(ev[self.K]), first

    def algorithmic_bytes(self, first):
        """Mean algorithmic bytes of the timed steps: each step's lengths and,
        per layer, the distinct experts its routing record shows."""
        import numpy as np

        from moe_persistent_decode_amd import sol
        if self.m.dense:  # one FFN per layer, no routing
            tot = [sol.step_bytes(self.m, self.lens_host + first + i, [1] * self.m.n_layers, self.fp8)
                   for i in range(self.K)]
            return float(np.mean(tot)), 1.0
        rt = self.route.cpu().numpy()
        tot = []
        for i in range(self.K):
            n_active = [len(np.unique(rt[i, l])) for l in range(self.m.n_layers)]
            assert min(n_active) >= 1 and rt[i].min() >= 0, "routing record incomplete"
            tot.append(sol.step_bytes(self.m, self.lens_host + first + i, n_active, self.fp8))
        return float(np.mean(tot)), float(np.mean([len(np.unique(rt[i, l])) for i in range(self.K)
                                                   for l in range(self.m.n_layers)]))

    def close(self):
        import torch
        self.dec.close()
        del self.pool
        torch.cuda.empty_cache()


OPNAMES = {1: "EMBED", 2: "QKV", 3: "ATTN (claimer)", 4: "RESIDUAL", 5: "O_PROJ", 6: "ROUTER (+TOPK)",
           8: "MOE_UP (claimer)", 9: "MOE_FUSED (claimer)", 10: "LM_HEAD"}


def op_trace(r, path, raw_path=None):
    """One traced megakernel step: per task its opcode, layer, workgroup and
    device timestamps (start, dependencies satisfied, end); summarised per
    opcode and, for two layers, as a phase timeline."""
    import numpy as np
    import torch

    import moe_persistent_decode_amd as mk
    r.dec.set_mode(mk.MODE_MEGAKERNEL)
    info = r.dec.schedule_info(r.B, r.hint + r.done)
    buf = torch.zeros((info.n_tasks, 8), dtype=torch.int32, device="cuda")
    r.dec.set_task_trace(buf, info.n_tasks)
    r.run(1)
    r.dec.sync(r.stream)
    r.dec.set_task_trace(None, 0)
    tr = buf.cpu().numpy().astype(np.int64) & 0xffffffff
    if raw_path:
        np.save(raw_path, tr)
    op, layer = tr[:, 0] & 0xff, (tr[:, 0] >> 8) & 0xff
    t0 = tr[:, 1].min()
    us = lambda k: (tr[:, k] - t0) / 100.0  # 100 MHz device clock
    start, waited, end = us(1), us(2), us(5)
    span = end.max()
    cmd = "python3 bench.py " + " ".join(sys.argv[1:])
    lines = [f"# Per-opcode time of one decode step: {r.wl.name}{' (FP8 feed-forward weights)' if r.fp8 else ''}", "",
             f"Command (on the MI355X box): `{cmd}`", "",
             f"One traced megakernel step (batch {r.B}); step span {span:.1f} us over {info.n_cus} workgroups.", "",
             "| opcode | tasks | mean wait (us) | mean run after wait (us) | workgroup-time share |",
             "|---|---:|---:|---:|---:|"]
    busy = (end - start).sum()
    for k in sorted(set(op.tolist())):
        m = op == k
        lines.append(f"| {OPNAMES.get(int(k), k)} | {int(m.sum())} | {(waited - start)[m].mean():.2f} | "
                     f"{(end - waited)[m].mean():.2f} | {(end - start)[m].sum() / busy:.1%} |")
    L = r.m.n_layers
    for l in sorted({1, L // 4 + (3 - (L // 4) % 4) % 4, L - 1} & set(range(L))):
        lines += ["", f"Layer {l} ({'full' if r.m.layer_window(l) == 0 else 'window'} attention): "
                  "first dependency satisfied / median / last end (us from step start)", "",
                  "| opcode | first waited | median waited | last end |", "|---|---:|---:|---:|"]
        for k in (6, 2, 3, 8, 9, 5, 4):
            m = (layer == l) & (op == k)
            if m.any():
                lines.append(f"| {OPNAMES[k]} | {waited[m].min():.1f} | {np.median(waited[m]):.1f} | {end[m].max():.1f} |")
    m = op == 10
    lines += ["", f"LM head: first waited {waited[m].min():.1f} us, last end {end[m].max():.1f} us."]
    open(path, "w").write("\n".join(lines) + "\n")
    log(f"[bench] per-opcode trace written to {path}")


def library_sha16():
    """Hash of the sources the decode step is built from (device code and the
    host scheduler): counter figures hold only for the code they measured."""
    import hashlib
    hs = hashlib.sha256()
    for f in ("mk_device.hip", "mk_host.cpp", "mk_internal.h", "mk_launch.h"):
        hs.update(open(os.path.join(ROOT, "moe_persistent_decode_amd", "csrc", f), "rb").read())
    return hs.hexdigest()[:16]


def counted_traffic(path, workload):
    """HBM bytes per launch of `workload` from the committed counter profile,
    or None when there is none for the current sources."""
    try:
        e = json.load(open(path)).get(workload)
        if e and e.get("library_sha256_16") == library_sha16():
            return e.get("hbm_bytes_per_launch")
    except (OSError, ValueError, AttributeError):
        pass
    return None


def percentiles(xs):
    """Median, 10th and 90th percentile of per-step times (ms)."""
    import numpy as np
    a = np.asarray(xs, np.float64)
    return {"median": round(float(np.median(a)), 4), "p10": round(float(np.percentile(a, 10)), 4),
            "p90": round(float(np.percentile(a, 90)), 4)}


def measure(wl, steps, warmup, ab, trace_path=None, raw_path=None, fp8=False):
    import moe_persistent_decode_amd as mk
    r = Run(wl, steps, warmup, 2 if ab else 1, fp8)
    ms, first = r.timed(mk.MODE_MEGAKERNEL, record=True)
    step_ms = ms / r.K
    bytes_avg, n_act = r.algorithmic_bytes(first)
    res = {"ms_per_step": step_ms, "tok_s": r.B * r.K / (ms / 1e3), "bytes": bytes_avg,
           "gbs": bytes_avg / (step_ms / 1e3) / 1e9, "experts_per_layer": n_act, "seq_len": r.hint,
           "lens": (int(r.lens_host.min()), int(r.lens_host.max()), float(r.lens_host.mean())),
           "step_ms": percentiles(r.step_ms)}
    log(f"[bench] {wl.name}{' fp8' if fp8 else ''} megakernel: {step_ms:.3f} ms/step, {res['tok_s']:.1f} tok/s, {res['gbs']:.0f} GB/s "
        f"({res['gbs'] / PEAK_GBS:.1%} of 8 TB/s), {n_act:.1f} experts per layer")
    if ab:
        ms_op, _ = r.timed(mk.MODE_KERNEL_PER_OP)
        res["kernel_per_op"] = {"ms_per_step": round(ms_op / r.K, 4), "tok_s": round(r.B * r.K / (ms_op / 1e3), 2),
                                "megakernel_speedup": round(ms_op / ms, 3), "step_ms": percentiles(r.step_ms)}
        log(f"[bench] {wl.name} kernel-per-op: {ms_op / r.K:.3f} ms/step -> megakernel {ms_op / ms:.2f}x")
    if trace_path:
        op_trace(r, trace_path, raw_path)
    bs = r.bs
    r.close()
    return res, bs


def stream_ceiling(gib=4, reps=10):
    """The streaming-read ceiling: GB/s of mk_stream_read over a buffer far
    larger than the last-level cache (median of `reps` timed reads)."""
    import numpy as np
    import torch

    import moe_persistent_decode_amd as mk
    buf = torch.empty(gib << 30, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    st = torch.cuda.current_stream()
    for _ in range(3):
        mk.stream_read(buf, st)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record(st)
    for i in range(reps):
        mk.stream_read(buf, st)
        ev[i + 1].record(st)
    torch.cuda.synchronize()
    ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]
    gbs = (gib << 30) / (float(np.median(ms)) / 1e3) / 1e9
    del buf
    torch.cuda.empty_cache()
    log(f"[bench] streaming-read ceiling: {gbs:.0f} GB/s ({gbs / PEAK_GBS:.1%} of 8 TB/s) over {gib} GiB")
    return {"gbs": round(gbs, 1), "frac_of_peak": round(gbs / PEAK_GBS, 4), "bytes": gib << 30, "reads": reps}


def measure_flushed(wl, steps, warmup):
    """One decode step at a time with the last-level cache evicted before each
    (a 1 GiB streaming read between steps, outside the timed events): for a
    model whose weights fit in the 256 MB cache, the HBM-bound time."""
    import numpy as np
    import torch

    import moe_persistent_decode_amd as mk
    r = Run(wl, steps, warmup, 2)
    flush = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
    ms_cached, first_c = r.timed(mk.MODE_MEGAKERNEL)
    r.run(r.W)
    r.dec.sync(r.stream)
    first = r.done
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(r.K)]
    for i, (a, b) in enumerate(pairs):
        mk.stream_read(flush, r.stream)
        a.record(r.stream)
        r.run(1, True, slot=i)
        b.record(r.stream)
    torch.cuda.synchronize()
    r.dec.sync(r.stream)
    ms = np.array([a.elapsed_time(b) for a, b in pairs])
    bytes_avg, n_act = r.algorithmic_bytes(first)
    med = float(np.median(ms))
    res = {"workload": wl.name, "steps": r.K, "step_ms": percentiles(ms), "tok_s": round(r.B / (med / 1e3), 2),
           "achieved_gbs": round(bytes_avg / (med / 1e3) / 1e9, 1),
           "frac": round(bytes_avg / (med / 1e3) / 1e9 / PEAK_GBS, 4), "algorithmic_bytes_per_launch": int(bytes_avg),
           "unflushed_ms_per_step": round(ms_cached / r.K, 4), "flush": "1 GiB streaming read before each step"}
    log(f"[bench] {wl.name} flushed: {med:.3f} ms/step median ({res['achieved_gbs']:.0f} GB/s, "
        f"{res['frac']:.1%} of 8 TB/s); unflushed {ms_cached / r.K:.3f} ms/step")
    del flush
    r.close()
    return res


ORDERS = {0: "shipped", 1: "qkv-first", 2: "attention-first"}
PLACEMENTS = {0: "tuned", 1: "round-robin", 2: "affinity"}


def ablation(path, steps, warmup):
    """The scheduler ablation (megakernel post, Chinese version, section on the
    task scheduler: wave orders and a dependency-affinity placement timed at
    batch 1, 2 and 4 with 8K contexts): tok/s of every combination, the same
    inputs and greedy decoding, and each one's logits against the shipped
    schedule's on the same step."""
    import numpy as np
    import torch

    import moe_persistent_decode_amd as mk
    from mkinputs import configs
    rows = []
    for name in ("full48_b1_8k", "full48_b2_8k", "full48_b4_8k"):
        wl = configs.WORKLOADS[name]
        runs = 1 + len(ORDERS) * len(PLACEMENTS)
        r = Run(wl, steps, warmup, runs)
        base = None
        for placement in PLACEMENTS:
            for order in ORDERS:
                r.dec.set_schedule_options(order, placement)
                ms, first = r.timed(mk.MODE_MEGAKERNEL)
                # one more step from the initial state (the first decode position
                # again: its K/V slot is rewritten with the same values, every
                # earlier slot is the untouched context): logits against the
                # shipped schedule's
                tok0, len0 = r.tokens.clone(), r.seq_lens.clone()
                r.tokens.copy_(torch.tensor(r.bs.tokens.numpy(), device="cuda"))
                r.seq_lens.copy_(torch.tensor(r.bs.seq_lens.numpy(), device="cuda"))
                r.dec.step(r.tokens, r.bt, r.seq_lens, r.hint + r.done, r.logits, stream=r.stream)
                r.dec.sync(r.stream)
                lg = r.logits.cpu().numpy()
                r.tokens.copy_(tok0)
                r.seq_lens.copy_(len0)
                if base is None:
                    base = lg
                d = float(np.abs(lg - base).max())
                rows.append((wl.batch, ORDERS[order], PLACEMENTS[placement], r.B * r.K / (ms / 1e3), ms / r.K, d,
                              bool(np.array_equal(np.argmax(lg, -1), np.argmax(base, -1)))))
                log(f"[ablation] B={wl.batch} {ORDERS[order]:15s} {PLACEMENTS[placement]:11s} "
                    f"{rows[-1][3]:8.1f} tok/s  {ms / r.K:.3f} ms/step  max|logits - shipped| {d:.2e}")
        r.close()
    lines = ["# Scheduler ablation: wave order and placement (48 layers, 8K context)", "",
             "Command (from the repository root on the MI355X box):", "", "```",
             f"python3 bench.py --ablation {os.path.basename(path)} --steps {steps} --warmup {warmup}", "```", "",
             "Megakernel decode rate per combination, greedy decoding from the same inputs "
             f"({steps} timed steps after {warmup} warm-up steps each). The last columns compare one "
             "step's logits with the shipped order and tuned placement on the same state (the fused "
             "MoE of at most 4 tokens groups the claimers' partial sums by their shares, so placements "
             "may differ in the last bits).", "",
             "| batch | wave order | placement | tok/s | ms/step | vs shipped + tuned | max abs logit diff | greedy equal |",
             "|---:|---|---|---:|---:|---:|---:|---|"]
    ref = {b: t for b, o, p, t, _, _, _ in rows if o == "shipped" and p == "tuned"}
    for b, o, p, t, ms, d, eq in rows:
        lines.append(f"| {b} | {o} | {p} | {t:.1f} | {ms:.3f} | {t / ref[b] - 1:+.1%} | {d:.1e} | {eq} |")
    open(path, "w").write("\n".join(lines) + "\n")
    log(f"[ablation] table written to {path}")


def search(path, workloads, n_random, steps, warmup):
    """The other schedulers of the megakernel post (Chinese version, section
    on the schedulers it tried): a greedy cost-model placement and a
    brute-force search over seeded random placements, against round-robin
    and the tuned placement. Every candidate is timed for `steps` steps; the
    five fastest random candidates, the cost model, round-robin and tuned are
    then timed again, interleaved, for four times as many steps (the first
    round's winner is biased upward by the selection). Each candidate's logits
    on one step from the initial state are compared with the tuned one's."""
    import numpy as np
    import torch

    import moe_persistent_decode_amd as mk
    from mkinputs import configs
    lines = ["# Schedule search: cost-model and random placements", "",
             "Command (from the repository root on the MI355X box):", "", "```",
             f"python3 bench.py --search {os.path.basename(path)} --search-workloads {','.join(workloads)} "
             f"--search-candidates {n_random} --steps {steps} --warmup {warmup}", "```", "",
             f"{n_random} random candidates (every wave over a seeded random permutation of the units) and the "
             "greedy cost-model placement (static tasks on the unit where a bytes-and-hops model says they finish "
             f"first), timed for {steps} steps each after {warmup} warm-up steps; the five fastest random "
             f"candidates, the cost model, round-robin and tuned then re-timed, interleaved, for {4 * steps} steps, "
             "three times (median shown). Logits of one step from the initial state against tuned's.", ""]
    for name in workloads:
        wl = configs.WORKLOADS[name]
        cands = [("tuned", mk.PLACE_TUNED, 0), ("round-robin", mk.PLACE_ROUND_ROBIN, 0),
                 ("cost model", mk.PLACE_COST_MODEL, 0)] + [(f"random {s}", mk.PLACE_RANDOM, s)
                                                            for s in range(1, n_random + 1)]
        runs = len(cands) + 3 * 8 * 4 + 2
        r = Run(wl, steps, warmup, runs)
        tok0, len0 = r.tokens.clone(), r.seq_lens.clone()

        def use(pl, seed):
            r.dec.set_schedule_options(0, pl)
            r.dec.set_placement_seed(seed if seed else 1)

        def logits_now():
            t_, l_ = r.tokens.clone(), r.seq_lens.clone()
            r.tokens.copy_(tok0)
            r.seq_lens.copy_(len0)
            r.dec.step(r.tokens, r.bt, r.seq_lens, r.hint + r.done, r.logits, stream=r.stream)
            r.dec.sync(r.stream)
            lg = r.logits.cpu().numpy()
            r.tokens.copy_(t_)
            r.seq_lens.copy_(l_)
            return lg

        first = {}
        base = None
        for label, pl, seed in cands:
            use(pl, seed)
            ms, _ = r.timed(mk.MODE_MEGAKERNEL)
            lg = logits_now()
            if base is None:
                base = lg
            first[label] = (ms / r.K, float(np.abs(lg - base).max()),
                            bool(np.array_equal(np.argmax(lg, -1), np.argmax(base, -1))))
        log(f"[search] {name}: " + ", ".join(f"{k} {v[0]:.3f}" for k, v in list(first.items())[:4]) + " ms ...")
        rand = sorted((k for k in first if k.startswith("random")), key=lambda k: first[k][0])[:5]
        final = ["tuned", "round-robin", "cost model"] + rand
        spec = {lab: (pl, sd) for lab, pl, sd in cands}
        K0, r.K = r.K, 4 * steps
        again = {k: [] for k in final}
        for _ in range(3):
            for k in final:
                use(*spec[k])
                ms, _ = r.timed(mk.MODE_MEGAKERNEL)
                again[k].append(ms / r.K)
        r.K = K0
        r.close()
        med = {k: float(np.median(v)) for k, v in again.items()}
        rr = med["round-robin"]
        allr = sorted(first[k][0] for k in first if k.startswith("random"))
        lines += [f"## {name} (batch {wl.batch})", "",
                  f"Random candidates, first round: best {allr[0]:.3f} ms, median {allr[len(allr) // 2]:.3f} ms, "
                  f"worst {allr[-1]:.3f} ms per step.", "",
                  "| placement | ms/step (re-timed, median of 3) | tok/s | vs round-robin | vs tuned | first round ms | "
                  "max abs logit diff vs tuned | greedy equal |", "|---|---:|---:|---:|---:|---:|---:|---|"]
        for k in final:
            lines.append(f"| {k} | {med[k]:.3f} | {wl.batch / (med[k] / 1e3):.1f} | {rr / med[k] - 1:+.1%} | "
                         f"{med['tuned'] / med[k] - 1:+.1%} | {first[k][0]:.3f} | {first[k][1]:.1e} | {first[k][2]} |")
        lines.append("")
        log(f"[search] {name}: re-timed " + ", ".join(f"{k} {v:.3f}" for k, v in med.items()))
    open(path, "w").write("\n".join(lines) + "\n")
    log(f"[search] table written to {path}")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the decode step "
              "runs on a single MI355X, with no collectives)", file=sys.stderr)
        sys.exit(2)
    import torch

    from mkinputs import configs, gen
    torch.cuda.set_device(0)
    if args.ablation:
        ablation(args.ablation, args.steps, args.warmup)
        return
    if args.search:
        search(args.search, args.search_workloads.split(","), args.search_candidates, args.steps, args.warmup)
        return
    wl = configs.WORKLOADS[args.workload]
    res, bs = measure(wl, args.steps, args.warmup, not args.no_ab, args.op_trace, args.op_trace_raw,
                      fp8=args.ffn_fp8)

    traffic = counted_traffic(args.traffic_json, wl.name + ("_fp8" if args.ffn_fp8 else ""))
    out = {
        "metric": "decode tok/s at batch 1 and 32, 8K ctx; HBM GB/s as % of MI355X peak",
        "value": round(res["tok_s"], 2),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16, fp8 e4m3 feed-forward weights" if args.ffn_fp8 else "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "seq_len": res["seq_len"],
                   "decode": "greedy, in-kernel advance"},
        "step_ms": res["step_ms"],
        "roofline": {"bound": "hbm", "achieved": round(res["gbs"], 1), "peak": PEAK_GBS, "unit": "GB/s",
                     "frac": round(res["gbs"] / PEAK_GBS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": int(res["bytes"]),
                     "kernel": f"mk_interp<{wl.model.head_dim}, 1{', true' if args.ffn_fp8 else ''}> "
                               "(one launch per step)"},
    }
    if "kernel_per_op" in res:
        out["kernel_per_op"] = res["kernel_per_op"]

    def summary(w, rr, k):
        d = {"workload": w.name, "batch": w.batch, "lengths": rr["lens"], "steps": k,
             "tok_s": round(rr["tok_s"], 2), "ms_per_step": round(rr["ms_per_step"], 4), "step_ms": rr["step_ms"],
             "achieved_gbs": round(rr["gbs"], 1), "frac": round(rr["gbs"] / PEAK_GBS, 4),
             "algorithmic_bytes_per_launch": int(rr["bytes"]),
             "experts_per_layer": round(rr["experts_per_layer"], 1)}
        if "kernel_per_op" in rr:
            d["kernel_per_op"] = rr["kernel_per_op"]
        return d

    bs_b = None
    if args.batch_workload != "none":
        wb = configs.WORKLOADS[args.batch_workload]
        kb = max(8, args.steps // 4)
        rb, bs_b = measure(wb, kb, min(args.warmup, 4), not args.no_ab)
        out["second_workload"] = summary(wb, rb, kb)
        out["second_workload"]["traffic"] = counted_traffic(args.traffic_json, wb.name)
    # the dense Llama-3.2-1B-shaped decoder on the same C ABI
    if args.dense_workload != "none":
        wd = configs.WORKLOADS[args.dense_workload]
        kd = max(8, args.steps // 2)
        rd, _ = measure(wd, kd, min(args.warmup, 4), not args.no_ab)
        out["dense_workload"] = summary(wd, rd, kd)
    # the same models with FP8 (E4M3) feed-forward weights, the rest bf16;
    # bytes and roofline fraction count the FP8 codes and scales
    if args.fp8_workloads != "none":
        out["fp8_weights"] = []
        for i, name in enumerate(args.fp8_workloads.split(",")):
            wf = configs.WORKLOADS[name]
            kf = max(8, args.steps // (4 if wf.batch > 4 else 2))
            rf, _ = measure(wf, kf, min(args.warmup, 4), False, args.fp8_op_trace if i == 0 else None, fp8=True)
            d = summary(wf, rf, kf)
            d["weights"] = "feed-forward FP8 E4M3 (per-hidden-unit float32 scales), other weights bf16"
            out["fp8_weights"].append(d)
    # long contexts: one sequence at 256K and four at 64K (the same model)
    if args.long_workloads != "none":
        out["long_context"] = []
        for name in args.long_workloads.split(","):
            wq = configs.WORKLOADS[name]
            kq = max(4, args.steps // 8)
            rq, _ = measure(wq, kq, min(args.warmup, 2), False)
            out["long_context"].append(summary(wq, rq, kq))

    if args.single_layer != "none":
        out["single_layer"] = measure_flushed(configs.WORKLOADS[args.single_layer], 16, 4)
    if not args.no_ceiling:
        out["stream_read_ceiling"] = stream_ceiling()

    if args.calibrate_copy:
        # a copy of known size: 256 MiB read and 256 MiB written per launch
        a = torch.ones(64 << 20, dtype=torch.int32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        log("[bench] copy calibration: 3 copies of 268435456 bytes")
        del a, b

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, bs)
        log(f"[bench] oracle on host: {out['cpu_baseline']}")
        if bs_b is not None:
            # one timed step at batch 32 (a step of the oracle there takes
            # about as long as the budget)
            out["second_workload"]["cpu_baseline"] = cpu_baseline(wb, bs_b, budget_s=0.0)
            log(f"[bench] oracle on host, {wb.name}: {out['second_workload']['cpu_baseline']}")

    print(json.dumps(out), flush=True)


def cpu_baseline(wl, bs, budget_s=10.0):
    """The oracle (test infrastructure) timed on the host for decode steps of
    the same workload: weights drawn on the GPU exactly as the timed run drew
    them, kept in host memory by a first, untimed step; then as many steps as
    fit in about `budget_s` seconds are timed."""
    import numpy as np

    from mkinputs import gen
    from oracle import decode as od
    m = wl.model
    W = gen.LazyWeights(m, wl.seed_weights, device="cuda")
    pool = gen.bf16_bits(gen.make_kv_pool(m, bs.n_pages, seed=wl.seed_kv, device="cuda"))
    bt = bs.block_tables.numpy()
    toks = bs.tokens.numpy()
    lens = bs.seq_lens.numpy().astype(np.int64)
    lg, _ = od.decode_step(m, W, pool, bt, toks, lens)
    n = 0
    t = time.time()
    while n < 1 or (time.time() - t < budget_s and n < 8):
        toks = od.greedy(lg)
        lens = lens + 1
        lg, _ = od.decode_step(m, W, pool, bt, toks, lens)
        n += 1
    dt = time.time() - t
    # the oracle's arithmetic runs in numpy's BLAS: its thread count is the
    # cores used; the host's CPU count is given beside it
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count()
    return {"value": round(wl.batch * n / dt, 4), "unit": "tok/s", "cores": cores, "host_cpus": os.cpu_count(),
            "kind": "oracle",
            "sample": f"{n} greedy decode steps of {wl.name} (batch {wl.batch}, from seq_len {int(bs.seq_lens.max())}) "
                      f"after one untimed step; weights resident in host memory; {dt:.1f} s"}


if __name__ == "__main__":
    main()
