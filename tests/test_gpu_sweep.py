"""GPU parity over a seeded sweep of random layer shapes, both precisions.

Each case draws M, N, the group count, the rank and the bias at random
(fixed seed), builds a layer with the tiny config's distributions (planted
outlier channels included), and runs the whole layer (kernel 1 then kernel
2, through the C ABI) against the oracle: codes and scales bit-exact, Y
within the stated bound and the per-element bound of the parity tests."""

import functools

import numpy as np
import pytest
import torch

import bit_quantized_diffusion_amd as bq
from tests import _cases as C
from tests.test_gpu_parity import assert_y_close, dev_bf16, device_layer, host_u16, say
from tests.test_gpu_mxfp4 import _mx_layer

pytestmark = pytest.mark.gpu


def _draw(n, k_step, max_groups, seed):
    """n shapes (M, K, N, rank, seed, bias) with K a multiple of k_step."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        M = int(rng.integers(1, 301))
        N = int(rng.integers(1, 401))
        K = k_step * int(rng.integers(1, max_groups + 1))
        rank = int(rng.choice([0, 16, 32, 48, 64]))
        rank = min(rank, 16 * (min(K, N) // 16))       # the ABI's rule: rank <= min(K, N)
        out.append((M, K, N, rank, 200 + i + (0 if k_step == 64 else 100), bool(rng.integers(0, 2))))
    return out


SWEEP_INT4 = _draw(16, 64, 32, 20261203)
SWEEP_MX = _draw(10, 128, 16, 20261204)


@functools.lru_cache(maxsize=None)
def _case(p):
    return C.small_case(*p)


@pytest.fixture(autouse=True)
def _require_device():
    assert bq.device_check(0), "gfx950 device required for the GPU tests"


@pytest.mark.parametrize("p", SWEEP_INT4, ids=lambda p: "M%dK%dN%dr%d" % p[:4])
def test_sweep_int4_layer(p):
    case = _case(p)
    say(f"sweep int4 {p}")
    pk = case["pk"]
    M = case["x"].shape[0]
    layer = device_layer(case)
    x = dev_bf16(case["x"])
    xq, xs, la = bq.quantize_act_lora_down(x, layer.smooth_inv, layer.lora_down, case["rank"])
    y = bq.linear(x, layer)
    torch.cuda.synchronize()
    ref = C.oracle_rows(case, np.arange(M))
    assert np.array_equal(xq.cpu().numpy(), ref["xq"])
    assert np.array_equal(host_u16(xs), ref["xs"].view(np.uint16))
    sl = C.int4_slack(ref, ref["xs"], pk["ws"], ref["t"], pk["l2"], case["bias"], t_from_kernel=True)
    assert_y_close(host_u16(y), ref["y"], "sweep int4", sl, ref["y64"])


@pytest.mark.parametrize("p", SWEEP_MX, ids=lambda p: "M%dK%dN%dr%d" % p[:4])
def test_sweep_mxfp4_layer(p):
    case = _case(p)
    pk = C.mx_pack(case)
    say(f"sweep mxfp4 {p}")
    M = case["x"].shape[0]
    layer = _mx_layer(case, pk)
    x = dev_bf16(case["x"])
    xq, xs, la = bq.quantize_act_lora_down(x, layer.smooth_inv, layer.lora_down, case["rank"], bq.MXFP4)
    y = bq.linear(x, layer)
    torch.cuda.synchronize()
    ref = C.mx_oracle_rows(case, np.arange(M))
    assert np.array_equal(xq.cpu().numpy(), ref["xq"])
    assert np.array_equal(xs.cpu().numpy(), ref["xs"])
    sl = C.mx_slack(ref["xq"], ref["xs"], pk["wq"], pk["ws"], ref["t"], pk["l2"], case["bias"], t_from_kernel=True)
    assert_y_close(host_u16(y), ref["y"], "sweep mxfp4", sl, ref["y64"])


def test_sweep_shapes_cover_the_edges():
    """The drawn shapes reach ragged tiles on both sides, short K loops and
    ranks 0 to 48 (a check of the draw itself, no device work)."""
    for sweep in (SWEEP_INT4, SWEEP_MX):
        assert any(p[0] % 128 for p in sweep) and any(p[2] % 128 for p in sweep)
    assert {p[3] for p in SWEEP_INT4 + SWEEP_MX} >= {0, 16, 32, 48}
    assert min(p[1] for p in SWEEP_INT4) <= 256
