"""GPU parity of the W4A16 comparison GEMM (4-bit weights, bf16
activations) through the C ABI against the W4A16 oracle.

Bar: Y within max|Y - Y_oracle| <= 1e-2 * max|Y_oracle| (fp32 accumulation
against fp64); bit-exact where every product and partial sum is exact in
fp32 (small integer activations, power-of-two group scales)."""

import functools

import numpy as np
import pytest
import torch

import bit_quantized_diffusion_amd as bq
import oracle as O
from tests import _cases as C
from tests.test_gpu_parity import assert_y_close, dev, dev_bf16, host_u16, say

pytestmark = pytest.mark.gpu

# (M, K, N, seed, bias)
SHAPES = [
    (256, 512, 512, 20, True),     # tiny config shape
    (300, 576, 200, 21, True),     # ragged M and N, odd group count
    (129, 256, 131, 22, False),    # odd N (element stores)
    (1, 64, 1, 23, True),          # one token, one channel, one group
    (64, 128, 64, 24, False),      # exactly the ring's two slots
    (520, 1024, 264, 25, True),
    (40, 4096, 272, 26, True),
]


@pytest.fixture(autouse=True)
def _require_device():
    assert bq.device_check(0), "gfx950 device required for the GPU tests"


@functools.lru_cache(maxsize=None)
def _case(p):
    M, K, N, seed, bias = p
    case = C.small_case(M, K, N, 0, seed, bias)
    wq, ws = O.pack_w4a16(case["w"])
    return case, wq, ws


def _run(case, wq, ws, rows=None):
    M, K = case["x"].shape
    N = wq.shape[0]
    b = None if case["bias"] is None else dev_bf16(case["bias"])
    y = bq.gemm_w4a16(dev_bf16(case["x"]), dev(wq), dev(ws), b, N)
    torch.cuda.synchronize()
    return host_u16(y)


@pytest.mark.parametrize("p", SHAPES, ids=lambda p: "M%dK%dN%d" % p[:3])
def test_w4a16_parity(p):
    case, wq, ws = _case(p)
    say(f"w4a16 {p}")
    got = _run(case, wq, ws)
    ref = O.w4a16_linear(case["x"], wq, ws, case["bias"])
    assert_y_close(got, ref["y"], "w4a16")


def test_w4a16_exact_products_bit_exact():
    """Integer activations in [-8, 8] and weights q * 2^e with e in [-4, 0]:
    every product and every fp32 partial sum is exact, so Y equals the
    oracle bit for bit whatever the summation order.  A weight, scale or
    activation taken from the wrong row, group or k shows here."""
    rng = np.random.default_rng(71)
    M, K, N = 200, 512, 136
    x = rng.integers(-8, 9, size=(M, K)).astype(np.float32)
    q = rng.integers(-7, 8, size=(N, K))
    q[:, ::64] = 7
    e = rng.integers(-4, 1, size=(N, K // 64))
    w = (q * np.exp2(np.repeat(e, 64, axis=1))).astype(np.float32)
    b = rng.integers(-4, 5, size=N).astype(np.float32)
    xb, wb, bb = O.f32_to_bf16_bits(x), O.f32_to_bf16_bits(w), O.f32_to_bf16_bits(b)
    wq, ws = O.pack_w4a16(wb)
    y = bq.gemm_w4a16(dev_bf16(xb), dev(wq), dev(ws), dev_bf16(bb), N)
    torch.cuda.synchronize()
    ref = O.w4a16_linear(xb, wq, ws, bb)
    assert np.array_equal(ref["y64"], x.astype(np.float64) @ w.T.astype(np.float64) + b)
    assert np.array_equal(host_u16(y), ref["y"])


def test_w4a16_output_buffer_reused():
    case, wq, ws = _case(SHAPES[1])
    M, K = case["x"].shape
    N = wq.shape[0]
    y = torch.full((M, N), 7.0, dtype=torch.bfloat16, device="cuda")
    out = bq.gemm_w4a16(dev_bf16(case["x"]), dev(wq), dev(ws), dev_bf16(case["bias"]), N, y=y)
    torch.cuda.synchronize()
    assert out.data_ptr() == y.data_ptr()
    assert_y_close(host_u16(y), O.w4a16_linear(case["x"], wq, ws, case["bias"])["y"], "w4a16 reuse")


def test_w4a16_full_size_fc1():
    """FLUX fc1 (4608 x 3072 -> 12288) in W4A16: sampled rows against the
    oracle, which dequantizes the whole weight once."""
    say("w4a16 full-size fc1: building case")
    case = C.named_case("fc1")
    wq, ws = O.pack_w4a16(case["w"])
    M = case["x"].shape[0]
    got = _run(case, wq, ws)
    rng = np.random.default_rng(6)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, M - 1], rng.choice(M, 27, replace=False)]))
    ref = O.w4a16_linear(case["x"][rows], wq, ws, case["bias"])
    assert_y_close(got[rows], ref["y"], "w4a16 fc1")


def test_w4a16_full_size_fc2():
    """FLUX fc2 (4608 x 12288 -> 3072, input bf16(GELU(fc1's Y))) in W4A16:
    sampled rows against the oracle."""
    say("w4a16 full-size fc2: building case")
    case = C.mlp_pair()[1]
    wq, ws = O.pack_w4a16(case["w"])
    M = case["x"].shape[0]
    got = _run(case, wq, ws)
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, M - 1], rng.choice(M, 27, replace=False)]))
    ref = O.w4a16_linear(case["x"][rows], wq, ws, case["bias"])
    assert_y_close(got[rows], ref["y"], "w4a16 fc2")
