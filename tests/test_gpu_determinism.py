"""Run-to-run behaviour of the two fused kernels.

Kernel 2 sums in a fixed order per output element (no atomics, no split of
K across workgroups), so on the same codes, scales and lora_act it writes
the same Y bit for bit, call after call: checked for the INT4 kernel's two
K-loop schedules (K below 8192 and from 8192 on) and for MXFP4.  Kernel 1's
codes and scales do not depend on any summation order and repeat bit for
bit; its lora_act adds the K slices' fp32 partials with atomics, so the
last bits may differ from call to call: checked against 2^-14 of its
largest magnitude (a real fault moves it by its own order)."""

import numpy as np
import pytest
import torch

import bit_quantized_diffusion_amd as bq
from tests import _cases as C
from tests.test_gpu_mxfp4 import _mx_layer
from tests.test_gpu_parity import dev_bf16, device_layer, host_u16, say

pytestmark = pytest.mark.gpu

CASES = [
    ("int4_fine", (520, 1024, 264, 16, 61, True), bq.INT4),
    ("int4_coarse", (300, 8192, 200, 32, 62, True), bq.INT4),
    ("mxfp4", (300, 1536, 200, 32, 63, True), bq.MXFP4),
]


@pytest.fixture(autouse=True)
def _require_device():
    assert bq.device_check(0), "gfx950 device required for the GPU tests"


@pytest.mark.parametrize("name,p,precision", CASES, ids=[c[0] for c in CASES])
def test_repeat_calls(name, p, precision):
    M, K, N, rank = p[:4]
    case = C.small_case(*p)
    layer = device_layer(case) if precision == bq.INT4 else _mx_layer(case, C.mx_pack(case))
    x = dev_bf16(case["x"])
    say(f"determinism {name} {p}")

    k1 = [bq.quantize_act_lora_down(x, layer.smooth_inv, layer.lora_down, rank, precision) for _ in range(3)]
    torch.cuda.synchronize()
    xq0, xs0, la0 = (t.cpu() for t in k1[0])
    for xq, xs, la in k1[1:]:
        assert torch.equal(xq.cpu(), xq0)
        assert torch.equal(xs.cpu().view(torch.uint8), xs0.view(torch.uint8))
        d = (la.cpu().double() - la0.double()).abs().max().item()
        assert d <= 2.0 ** -14 * la0.double().abs().max().item(), f"lora_act moved by {d}"

    xq, xs, la = k1[0]
    ys = [bq.gemm_w4a4_lora_up(xq, xs, layer.wq, layer.ws, la, layer.lora_up, layer.bias, M, N, K, rank, precision)
          for _ in range(4)]
    torch.cuda.synchronize()
    y0 = host_u16(ys[0])
    for i, y in enumerate(ys[1:], 1):
        assert np.array_equal(host_u16(y), y0), f"call {i} differs from call 0"
