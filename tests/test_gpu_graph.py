"""The fused layer under HIP-graph capture.

The two hot calls allocate nothing and clear lora_act with a kernel, not a
memset, so a caller can capture them into a graph.  Each case captures the
layer (both kernels) into a torch CUDA graph, replays it several times with
other eager work between the replays (a different layer on the same stream
and a host synchronization), and checks every replay against the oracle on
that replay's input with the parity tests' bounds (the stated one and the
per-element one).  The input is rewritten between replays, so a replay
that reused stale data would fail.  The eager call is checked the same way
(kernel 1 sums lora_act with atomics, so two runs need not agree bit for
bit: a last-bit change of an fp32 partial can flip its bf16 rounding in the
up projection)."""

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


def _layer(precision, p):
    case = C.small_case(*p)
    if precision == bq.INT4:
        return case, device_layer(case)
    return case, _mx_layer(case, C.mx_pack(case))


@pytest.mark.parametrize("precision", [bq.INT4, bq.MXFP4], ids=["int4", "mxfp4"])
def test_layer_graph_replays_match_eager(precision):
    p = (300, 1024, 200, 32, 41, True)
    case, layer = _layer(precision, p)
    _, other = _layer(precision, (64, 512, 136, 16, 42, False))
    say(f"graph {p} precision {precision}")
    x_static = dev_bf16(case["x"])
    rng = np.random.default_rng(7)
    inputs = [x_static.clone()] + [
        (x_static.float() * torch.from_numpy(rng.uniform(0.5, 2.0, x_static.shape[1]).astype(np.float32)).cuda())
        .to(torch.bfloat16) for _ in range(3)]
    x_other = dev_bf16(C.small_case(64, 512, 136, 16, 42, False)["x"])

    # warm up on a side stream, then capture
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        bq.linear(x_static, layer)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        y_static = bq.linear(x_static, layer)
    torch.cuda.synchronize()

    for i, x in enumerate(inputs):
        x_static.copy_(x)
        g.replay()
        bq.linear(x_other, other)                  # eager work between the replays
        torch.cuda.synchronize()
        want = bq.linear(x, layer)
        torch.cuda.synchronize()
        xb = host_u16(x)
        M = xb.shape[0]
        if precision == bq.INT4:
            pk = case["pk"]
            ref = C.oracle_rows(case, np.arange(M), x_bits=xb)
            sl = C.int4_slack(ref, ref["xs"], pk["ws"], ref["t"], pk["l2"], case["bias"], t_from_kernel=True)
        else:
            pk = C.mx_pack(case)
            ref = C.mx_oracle_rows(case, np.arange(M), x_bits=xb)
            sl = C.mx_slack(ref["xq"], ref["xs"], pk["wq"], pk["ws"], ref["t"], pk["l2"], case["bias"],
                            t_from_kernel=True)
        assert_y_close(host_u16(y_static), ref["y"], f"graph replay {i}", sl, ref["y64"])
        assert_y_close(host_u16(want), ref["y"], f"eager call {i}", sl, ref["y64"])
