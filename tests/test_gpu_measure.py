"""The measurement entry point (include/moe_bench.h) runs and its FLOP count
follows its definition; it is no step of the layer, so there is no oracle."""
import numpy as np
import pytest
import torch

from gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    from dropless_moe_expert_amd import ops as o
    o.load_library()
    return o


@pytest.mark.parametrize("random_operands", [True, False])
def test_mfma_ceiling_runs(ops, random_operands):
    say("mfma ceiling", random_operands)
    dev = torch.device("cuda")
    sink, flops = ops.bench_mfma_ceiling(random_operands, 8, 3, dev)
    torch.cuda.synchronize()
    assert flops == 3 * 8 * 8 * 32 * 2 * 16 * 16 * 32
    s = sink.cpu().numpy()
    assert s.shape == (3 * 512,) and np.isfinite(s).all()
    if not random_operands:
        # ones times ones: every accumulator element is 8 rounds x 32 products
        assert np.all(s == 2 * 8 * 32 * 4 * 8)
