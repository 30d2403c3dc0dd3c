"""GPU parity of the dense sequential model (the HIP path through the C ABI
vs the oracle): attention added to the residual stream, a second RMSNorm, the
SwiGLU FFN in 16-row slices (gate/up, SiLU-and-multiply and down per slice on
one unit) added in turn, and a head tied to the embedding.

Cases: the tiny dense model at batch 1, 2 and 4 over ragged contexts, both
the megakernel and the kernel-per-op variant, four teacher-forced steps with
every row's logits, greedy token and appended K/V compared; the Llama-3.2-1B
shaped model (16 layers, 8K context) at batch 1 with the kernel feeding itself
for four steps, and at batch 4 over ragged contexts for two. The LM head is
margin-repaired (tests.harness.lm_repair_hook) so every greedy token is
compared exactly.
"""
import pytest

from mkinputs import configs
from tests.test_gpu_batch import _run as run_batch
from tests.test_gpu_full import _run as run_full

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("B,lo,hi,seed", [(1, 129, 130, 61), (2, 30, 170, 62), (4, 20, 150, 63)])
def test_tiny_dense_batches(B, lo, hi, seed, mode):
    run_batch(B, lo, hi, seed, mode, cfg=configs.TINY_DENSE)


def test_tiny_dense_every_schedule_is_bit_identical():
    """The dense FFN's slices are shared equally over all units and summed in
    unit order, so the two schedule variants give the same bits."""
    import numpy as np
    a = run_batch(2, 30, 170, 64, 0, cfg=configs.TINY_DENSE)
    b = run_batch(2, 30, 170, 64, 1, cfg=configs.TINY_DENSE)
    for s, (x, y) in enumerate(zip(a, b)):
        assert np.array_equal(x, y), s


def test_llama1b_b1_8k_megakernel():
    """Four greedy steps of the dense benchmark configuration, the kernel
    writing each step's token and length for the next."""
    run_full(configs.WORKLOADS["llama1b_b1_8k"], 4, 0, stages=False, advance=True)


def test_llama1b_b4_ragged():
    run_full(configs.WORKLOADS["llama1b_b4_ragged"], 2, 0, stages=False)
