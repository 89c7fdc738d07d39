"""The split-K schedule of the fused INT4 GEMM (svdq_gemm_w4a4_lora_up_ws).

Shapes whose tiles leave most workgroup slots empty and whose K loop is
long: the workspace size is non-zero, the split result meets the parity
bounds against the oracle, as does the single-pass schedule on the same
inputs, and repeated split calls agree bit for bit (fixed summation order).
A workspace smaller than the size asked for runs the single-pass schedule,
whose output is then that of the entry point without a workspace."""

import numpy as np
import pytest
import torch

import bit_quantized_diffusion_amd as bq
from tests import _cases as C
from tests.test_gpu_parity import assert_y_close, dev_bf16, device_layer, host_u16, say

pytestmark = pytest.mark.gpu

# (M, K, N, rank, seed, bias): tiles x stages -> splits on a 256-CU part
SHAPES = [
    (136, 8192, 144, 16, 7, True),      # 4 tiles, 64 stages -> 8 splits of 8
    (72, 8256, 136, 32, 8, True),       # odd group count: 65 stages -> 8 splits of 9, the last 2
    (40, 4096, 272, 16, 12, True),      # 3 tiles, 32 stages -> 4 splits
    (33, 8192, 131, 16, 11, True),      # ragged M and N
    (300, 2048, 200, 32, 13, False),    # 6 tiles, 16 stages -> 2 splits, no bias
    (700, 3072, 520, 32, 14, True),     # 30 tiles, 24 stages -> 3 splits
]


@pytest.fixture(autouse=True)
def _require_device():
    assert bq.device_check(0), "gfx950 device required for the GPU tests"


@pytest.mark.parametrize("p", SHAPES, ids=lambda p: "M%dK%dN%dr%d" % p[:4])
def test_split_k_against_oracle_and_single_pass(p):
    M, K, N, rank = p[:4]
    case = C.small_case(*p)
    pk = case["pk"]
    say(f"split-K {p}")
    nbytes = bq.gemm_workspace_size(M, N, K)
    assert nbytes > 0
    layer = device_layer(case)
    x = dev_bf16(case["x"])
    xq, xs, la = bq.quantize_act_lora_down(x, layer.smooth_inv, layer.lora_down, rank)

    def gemm(ws):
        return bq.gemm_w4a4_lora_up(xq, xs, layer.wq, layer.ws, la, layer.lora_up, layer.bias, M, N, K, rank,
                                    workspace=ws)

    ws = torch.empty((nbytes,), dtype=torch.uint8, device=x.device)
    y_split = [gemm(ws) for _ in range(3)]
    y_plain = gemm(None)
    y_small_ws = gemm(torch.empty((nbytes - 16,), dtype=torch.uint8, device=x.device))
    torch.cuda.synchronize()

    ref = C.oracle_rows(case, np.arange(M))
    sl = C.int4_slack(ref, ref["xs"], pk["ws"], ref["t"], pk["l2"], case["bias"], t_from_kernel=True)
    assert_y_close(host_u16(y_split[0]), ref["y"], "split-K", sl, ref["y64"])
    assert_y_close(host_u16(y_plain), ref["y"], "single pass", sl, ref["y64"])
    for y in y_split[1:]:
        assert np.array_equal(host_u16(y), host_u16(y_split[0]))
    assert np.array_equal(host_u16(y_small_ws), host_u16(y_plain))


def test_workspace_size_rules():
    """No split where the grid already fills the device, where the K loop is
    short, or for MXFP4; the per-GPU share of FLUX's fc2 splits."""
    assert bq.gemm_workspace_size(4608, 12288, 3072) == 0      # fc1: 3456 tiles
    assert bq.gemm_workspace_size(4608, 3072, 12288) == 0      # fc2: 864 tiles
    assert bq.gemm_workspace_size(256, 512, 512) == 0          # 4 stages
    assert bq.gemm_workspace_size(576, 3072, 12288, bq.MXFP4) == 0
    assert bq.gemm_workspace_size(576, 12288, 3072) == 0       # fc1's share: 480 tiles
    n = bq.gemm_workspace_size(576, 3072, 12288)                # fc2's share: 120 tiles, 96 stages
    assert n > 0 and n % (120 * 65536) == 0
