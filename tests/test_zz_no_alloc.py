"""svdq_unfused_linear_noalloc (the unfused layer with its intermediates in
the library's own device array) against svdq_unfused_linear, the same
layer with caller-allocated workspace: two calls in a row, the second with
a smaller input, so the second call runs on what the first left in the
shared array.  Both outputs are also held to the per-element bound against
the oracle."""

import numpy as np
import pytest
import torch

import bit_quantized_diffusion_amd as bq
from tests import _cases as C
from tests.test_gpu_parity import assert_y_close, dev_bf16, device_layer, host_u16, say

pytestmark = pytest.mark.gpu

# (M, K, N, rank, seed, bias): the first call is the larger one
CALLS = [(1000, 3072, 520, 32, 31, True), (129, 192, 131, 48, 32, False)]


def _check_one(p):
    case = C.small_case(*p)
    pk = case["pk"]
    M = case["x"].shape[0]
    say(f"no-alloc unfused {p}")
    layer = device_layer(case)
    x = dev_bf16(case["x"])
    y_ref_path = bq.unfused_linear(x, layer)
    y = torch.full((M, layer.N), float("nan"), dtype=torch.bfloat16, device="cuda")
    bq.unfused_linear_noalloc(x, layer, y)
    torch.cuda.synchronize()
    ya, yb = host_u16(y), host_u16(y_ref_path)
    assert np.all(np.isfinite(y.float().cpu().numpy()))
    assert_y_close(ya, yb, "no-alloc vs unfused_linear")
    ref = C.oracle_rows(case, np.arange(M))
    sl = C.int4_slack(ref, ref["xs"], pk["ws"], ref["t"], pk["l2"], case["bias"], t_from_kernel=True)
    sl = sl + 0.5 * C.ulp_bf16(np.abs(ref["acc"]) + sl)
    assert_y_close(ya, ref["y"], "no-alloc vs oracle", sl, ref["y64"])
    assert_y_close(yb, ref["y"], "unfused vs oracle", sl, ref["y64"])


def test_noalloc_matches_unfused_two_calls():
    assert bq.device_check(0)
    for p in CALLS:
        _check_one(p)
