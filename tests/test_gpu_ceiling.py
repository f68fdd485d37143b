"""The MFMA ceiling measurement (iris_mfma_ceiling): both operand modes run
and report a rate and a clock in a plausible range for one MI355X, and
random operands are no faster than constant ones."""
import math

import pytest
import torch

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import gemm_collective_tile_amd as il
else:
    il = None


def test_mfma_ceiling_both_modes():
    const_t, const_m = il.iris_mfma_ceiling(random_operands=False, iters=50000)
    rand_t, rand_m = il.iris_mfma_ceiling(random_operands=True, iters=50000)
    for t, m in ((const_t, const_m), (rand_t, rand_m)):
        assert math.isfinite(t) and 200.0 < t < 2600.0, t  # the dense fp16 peak is 2500
        assert math.isfinite(m) and 100.0 < m < 2600.0, m
    assert rand_t <= 1.05 * const_t, (rand_t, const_t)
