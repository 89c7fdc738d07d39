"""Two layers on two streams at once.

The fused calls keep no state between calls and take every buffer from
the caller, so layers launched on different streams may overlap on the
device.  Two different layers (one INT4, one MXFP4) are launched
alternately on two side streams, several times each, with no host
synchronization between the launches; every output is then checked
against the oracle with the parity bounds."""

import numpy as np
import pytest
import torch

import bit_quantized_diffusion_amd as bq
from tests import _cases as C
from tests.test_gpu_mxfp4 import _mx_layer
from tests.test_gpu_parity import assert_y_close, dev_bf16, device_layer, host_u16, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _require_device():
    assert bq.device_check(0), "gfx950 device required for the GPU tests"


def test_two_streams_interleaved():
    pa = (520, 1024, 264, 16, 51, True)
    pb = (300, 1536, 200, 32, 52, True)
    ca, cb = C.small_case(*pa), C.small_case(*pb)
    pkb = C.mx_pack(cb)
    la, lb = device_layer(ca), _mx_layer(cb, pkb)
    xa, xb = dev_bf16(ca["x"]), dev_bf16(cb["x"])
    say(f"streams {pa} int4 / {pb} mxfp4")
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    outs_a, outs_b = [], []
    for _ in range(4):
        with torch.cuda.stream(sa):
            outs_a.append(bq.linear(xa, la))
        with torch.cuda.stream(sb):
            outs_b.append(bq.linear(xb, lb))
    torch.cuda.synchronize()
    ref_a = C.oracle_rows(ca, np.arange(pa[0]))
    sl_a = C.int4_slack(ref_a, ref_a["xs"], ca["pk"]["ws"], ref_a["t"], ca["pk"]["l2"], ca["bias"], t_from_kernel=True)
    ref_b = C.mx_oracle_rows(cb, np.arange(pb[0]))
    sl_b = C.mx_slack(ref_b["xq"], ref_b["xs"], pkb["wq"], pkb["ws"], ref_b["t"], pkb["l2"], cb["bias"], t_from_kernel=True)
    for i, (ya, yb) in enumerate(zip(outs_a, outs_b)):
        assert_y_close(host_u16(ya), ref_a["y"], f"stream A call {i}", sl_a, ref_a["y64"])
        assert_y_close(host_u16(yb), ref_b["y"], f"stream B call {i}", sl_b, ref_b["y64"])
