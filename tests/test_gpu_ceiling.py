"""The matrix-core ceiling kernel used by the measurement: it runs for both
operand formats, and every workgroup (same operand bits) returns the same
finite, non-zero checksum."""

import numpy as np
import pytest
import torch

import bit_quantized_diffusion_amd as bq

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("precision", [bq.INT4, bq.MXFP4], ids=["fp8", "fp4"])
def test_mfma_ceiling_runs(precision):
    assert bq.device_check(0)
    ops, out = bq.mfma_ceiling(precision, blocks=8, iters=16)
    torch.cuda.synchronize()
    v = out.cpu().numpy()
    assert ops == 8 * 4 * 8 * 16 * 131072
    assert np.all(np.isfinite(v)) and v[0] != 0
    assert np.all(v == v[0])
