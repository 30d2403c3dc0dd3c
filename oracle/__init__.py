"""Oracle: a plain, slow CPU decode step of the parallel-transformer MoE model.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import or run anything in this package. The HIP library
never calls it, links it or shares code with it; the two meet only through the
seeded inputs of `mkinputs`.

What it computes is the plain definition of one decode step (the megakernel
post, section "Where the speedup comes from", is explicit that tasks, schedules
and placement change only timing, never the result), written out layer by
layer in numpy at float32 (or float64) from bf16 weights and a bf16 paged KV
cache. Every function cites the passage it follows. Readings of passages that
are silent or garbled are listed in the module docstring of `oracle.decode`.

Pins (tests/test_oracle_pins.py, run with -m "not gpu") tie each function to
something other than itself: closed forms, invariants, library special cases,
brute force on tiny inputs, and an independent full-sequence recomputation.
"""
from .decode import (  # noqa: F401
    bf16_to_float,
    float_to_bf16_rne,
    rmsnorm,
    rope,
    silu,
    attention_one_head,
    router_topk,
    expert_ffn,
    decode_step,
    greedy,
    StepTrace,
    e4m3_to_float,
    fp8_ffn_weights,
    ffn_weights,
)
