"""GPU parity with FP8 feed-forward weights (the post's roadmap of narrower
weight types, Chinese version, section "下一步"): OCP E4M3 codes with one
float32 scale per hidden unit for its gate column, up column and down row,
the other weights bf16.

The input generator quantizes the drawn bf16 FFN weights once; the HIP path
and the oracle read the same codes and scales (the oracle decodes them from
the format's fields in float64). Cases, every row and step compared as in
the bf16 tests (logits within 3e-2 max abs and 1e-2 relative L2, greedy
tokens and every layer's top-k set identical, margins repaired):
- the tiny MoE model at batch 1, 2 and 4 (the fused MoE path) and at 8, 17
  and 32 (the claiming MoE, which an FP8 model runs at every batch above 4)
  over ragged contexts, both the megakernel and the kernel-per-op variant,
  and with a 48-token window on layer 0;
- the tiny dense model at batch 1 and 4;
- full size: the one-layer model at 8K (three steps) and at batch 32 with
  ragged 512..16384 contexts, the 48-layer model at batch 1 and 8K with the
  kernel advancing tokens itself and at batch 32 ragged (two steps each), and
  the Llama-3.2-1B-shaped dense model at batch 1 and 8K (two steps).
"""
import pytest

from mkinputs import configs
from tests.test_gpu_batch import _run as run_batch
from tests.test_gpu_full import _run as run_full

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("B,lo,hi,seed", [(1, 129, 130, 301), (2, 30, 170, 302), (4, 20, 150, 303)])
def test_tiny_fp8_batches(B, lo, hi, seed, mode):
    run_batch(B, lo, hi, seed, mode, fp8=True)


def test_tiny_window_fp8():
    run_batch(4, 8, 160, seed=310, mode=0, cfg=configs.TINY_WIN, fp8=True)


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("B,lo,hi,seed", [(8, 20, 150, 331), (17, 1, 64, 332), (32, 16, 200, 333)])
def test_tiny_fp8_claiming_batches(B, lo, hi, seed, mode):
    """Above 4 sequences an FP8 model runs the claiming MoE at every batch:
    one row tile at 8 and 17 (the second only for experts past 16 tokens),
    two at 32."""
    run_batch(B, lo, hi, seed, mode, fp8=True)


@pytest.mark.parametrize("B", [8, 32])
def test_tiny_window_fp8_claiming(B):
    run_batch(B, 8, 160, seed=340 + B, mode=0, cfg=configs.TINY_WIN, fp8=True)


@pytest.mark.parametrize("B,lo,hi,seed", [(1, 129, 130, 321), (4, 20, 150, 322)])
def test_tiny_dense_fp8(B, lo, hi, seed):
    run_batch(B, lo, hi, seed, 0, cfg=configs.TINY_DENSE, fp8=True)


def test_layer1_b1_8k_fp8():
    run_full(configs.WORKLOADS["layer1_b1_8k"], 3, 0, stages=False, fp8=True)


def test_full48_b1_8k_fp8():
    run_full(configs.WORKLOADS["full48_b1_8k"], 2, 0, stages=False, advance=True, fp8=True)


def test_layer1_b32_ragged_fp8():
    run_full(configs.WORKLOADS["layer1_b32_ragged"], 2, 0, stages=False, fp8=True)


def test_full48_b32_ragged_fp8():
    run_full(configs.WORKLOADS["full48_b32_ragged"], 2, 0, stages=False, fp8=True)


def test_llama1b_b1_8k_fp8():
    run_full(configs.WORKLOADS["llama1b_b1_8k"], 2, 0, stages=False, fp8=True)
