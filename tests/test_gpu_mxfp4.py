"""GPU parity of the MXFP4 variant (OCP Microscaling FP4: E2M1 codes, one
E8M0 scale per 32 k) through the C ABI against the MXFP4 oracle.

Bar: codes and scale bytes bit-exact; the fp32 down projection within
rtol 1e-3; Y within max|Y - Y_oracle| <= 1e-2 * max|Y_oracle|."""

import functools

import numpy as np
import pytest
import torch

import bit_quantized_diffusion_amd as bq
import oracle as O
from tests import _cases as C
from tests.test_gpu_parity import Y_TOL, assert_y_close, dev, dev_bf16, host_u16, say

pytestmark = pytest.mark.gpu

# (M, K, N, rank, seed, bias); K % 128 == 0 for MXFP4
SMALL_MX = [
    (256, 512, 512, 16, 10, False),   # tiny config shape
    (300, 640, 200, 32, 11, True),    # ragged M, 5 pipeline stages
    (129, 256, 131, 48, 12, True),    # odd N (element stores), 2 stages
    (1, 128, 1, 0, 13, True),         # single token and channel, one stage, rank 0
    (64, 384, 64, 64, 14, False),     # exactly the ring's 3 stages
    (520, 1024, 264, 16, 15, True),
    (40, 4096, 272, 256, 16, True),   # largest rank
    (70, 384, 131, 32, 17, True),     # rank 32 (up projection via LDS), odd N: bias from memory
    (65, 256, 34, 32, 18, True),      # rank 32, ragged even N: bias via LDS
]


@functools.lru_cache(maxsize=None)
def _mx_small(p):
    case = C.small_case(*p)
    return case, C.mx_pack(case)


def _mx_layer(case, pk):
    r = case["rank"]
    return bq.PackedLinear(
        K=case["x"].shape[1], N=pk["wq"].shape[0], rank=r, precision=bq.MXFP4,
        smooth_inv=dev(pk["smooth_inv"]),
        lora_down=dev_bf16(pk["l1"].T) if r else None,
        lora_up=dev_bf16(pk["l2"].T) if r else None,
        wq=dev(pk["wq"]), ws=dev(pk["ws"]),
        bias=None if case["bias"] is None else dev_bf16(case["bias"]))


@pytest.fixture(autouse=True)
def _require_device():
    assert bq.device_check(0), "gfx950 device required for the GPU tests"


@pytest.mark.parametrize("p", SMALL_MX, ids=lambda p: "M%dK%dN%dr%d" % p[:4])
def test_mx_k1_parity(p):
    case, pk = _mx_small(p)
    say(f"mx k1 {p}")
    r = case["rank"]
    layer = _mx_layer(case, pk)
    xq, xs, la = bq.quantize_act_lora_down(dev_bf16(case["x"]), layer.smooth_inv, layer.lora_down, r,
                                           bq.MXFP4)
    torch.cuda.synchronize()
    ref = O.mx_quantize_act_lora_down(case["x"], pk["smooth_inv"], pk["l1"])
    assert np.array_equal(xq.cpu().numpy(), ref["xq"])
    assert np.array_equal(xs.cpu().numpy(), ref["xs"])
    if r:
        t = ref["t"]
        got = la.cpu().numpy().astype(np.float64)
        assert np.allclose(got, t, rtol=1e-3, atol=1e-4 * np.max(np.abs(t)))


def test_mx_k1_edge_values():
    """Block magnitudes across the whole bf16 range (subnormal blocks whose
    exponent clamps at -127, the largest finite values), exact ties between
    E2M1 neighbours, values that round to zero with a negative sign, the
    saturation band above 6 * 2^e and all-zero blocks."""
    rng = np.random.default_rng(199)
    M, K = 96, 1024
    x = np.zeros((M, K), np.float32)
    for m in range(M):
        e = -133 + (m * 260) // M                    # block exponents 2^-133 .. 2^127
        row = rng.standard_normal(K) * 2.0 ** e
        if m % 5 == 1:                               # midpoints of the E2M1 grid after scaling
            mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
            row = rng.choice(mids, K) * rng.choice([-1.0, 1.0], K) * 2.0 ** e
            row[::32] = 6.0 * 2.0 ** e               # amax pins the block exponent to e
        if m % 7 == 2:
            row[64:96] = 0.0
        if m % 11 == 3:                              # tiny negatives next to a large value
            row[:32] = -rng.uniform(0, 0.2, 32) * 2.0 ** e
            row[0] = 4.0 * 2.0 ** e
        if m % 13 == 4:                              # values between 6 and 8 times the scale
            row[32:64] = rng.uniform(6.0, 7.99, 32) * 2.0 ** e * rng.choice([-1.0, 1.0], 32)
        x[m] = np.clip(row, -3.3e38, 3.3e38).astype(np.float32)
    xb = O.f32_to_bf16_bits(x)
    sinv = np.ones(K, np.float32)
    xq, xs, _ = bq.quantize_act_lora_down(dev_bf16(xb), dev(sinv), None, 0, bq.MXFP4)
    torch.cuda.synchronize()
    ref = O.mx_quantize_act_lora_down(xb, sinv, np.zeros((K, 0), np.uint16))
    assert np.array_equal(xs.cpu().numpy(), ref["xs"])
    assert np.array_equal(xq.cpu().numpy(), ref["xq"])


@pytest.mark.parametrize("p", SMALL_MX, ids=lambda p: "M%dK%dN%dr%d" % p[:4])
def test_mx_k2_parity(p):
    case, pk = _mx_small(p)
    say(f"mx k2 {p}")
    r = case["rank"]
    M, K = case["x"].shape
    N = pk["wq"].shape[0]
    ref = C.mx_oracle_rows(case, np.arange(M))
    layer = _mx_layer(case, pk)
    la = dev(ref["t"].astype(np.float32)) if r else None
    y = bq.gemm_w4a4_lora_up(dev(ref["xq"]), dev(ref["xs"]), layer.wq, layer.ws, la, layer.lora_up,
                             layer.bias, M, N, K, r, bq.MXFP4)
    torch.cuda.synchronize()
    sl = C.mx_slack(ref["xq"], ref["xs"], pk["wq"], pk["ws"], ref["t"], pk["l2"], case["bias"], t_from_kernel=False)
    assert_y_close(host_u16(y), ref["y"], "mx k2", sl, ref["y64"])


@pytest.mark.parametrize("shape", [(133, 768, 136), (260, 768, 132)], ids=["ragged", "rows4"])
@pytest.mark.parametrize("spread", [(120, 134), (100, 150), (0, 0)], ids=["near1", "wide", "zero"])
def test_mx_k2_block_scales(spread, shape):
    """Random codes with an independent random scale byte per 32-block of
    every row: a scale applied to the wrong block, row or lane half shows
    as a large error (checked per output row against that row's largest
    value).  (0, 0): every scale is 2^-127 and every product underflows.
    Row counts that are multiples of 4 load their scales as dwords of 4
    rows, the others byte by byte at the ragged edge."""
    lo, hi = spread
    say(f"mx k2 block scales {spread} {shape}")
    rng = np.random.default_rng([78, lo, hi])
    M, K, N = shape
    codes_x = rng.integers(0, 16, size=(M, K)).astype(np.uint8)
    codes_w = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    sx = rng.integers(lo, hi + 1, size=(K // 32, M)).astype(np.uint8)
    sw = rng.integers(lo, hi + 1, size=(K // 32, N)).astype(np.uint8)
    xq = (codes_x[:, 0::2] | (codes_x[:, 1::2] << 4)).astype(np.uint8)
    wq = (codes_w[:, 0::2] | (codes_w[:, 1::2] << 4)).astype(np.uint8)
    ref = O.mx_gemm_lora_up(xq, sx, wq, sw, np.zeros((M, 0)), np.zeros((0, N), np.uint16), None)
    y = bq.gemm_w4a4_lora_up(dev(xq), dev(sx), dev(wq), dev(sw), None, None, None, M, N, K, 0, bq.MXFP4)
    torch.cuda.synchronize()
    yb = host_u16(y)
    if hi == 0:
        assert np.all(O.bf16_bits_to_f32(yb) == 0)
        return
    sl = C.mx_slack(xq, sx, wq, sw, np.zeros((M, 0)), np.zeros((0, N), np.uint16), None, t_from_kernel=False)
    assert_y_close(yb, ref["y"], "mx block scales", sl, ref["y64"])
    got = O.bf16_bits_to_f32(yb).astype(np.float64)
    want = ref["y64"]
    row_err = np.max(np.abs(got - want), axis=1)
    row_max = np.max(np.abs(want), axis=1)
    assert np.all(row_err <= Y_TOL * row_max)


@pytest.mark.parametrize("p", SMALL_MX, ids=lambda p: "M%dK%dN%dr%d" % p[:4])
def test_mx_layer_end_to_end(p):
    case, pk = _mx_small(p)
    say(f"mx layer {p}")
    M = case["x"].shape[0]
    ref = C.mx_oracle_rows(case, np.arange(M))
    y = bq.linear(dev_bf16(case["x"]), _mx_layer(case, pk))
    torch.cuda.synchronize()
    sl = C.mx_slack(ref["xq"], ref["xs"], pk["wq"], pk["ws"], ref["t"], pk["l2"], case["bias"], t_from_kernel=True)
    assert_y_close(host_u16(y), ref["y"], "mx layer", sl, ref["y64"])


def test_mx_full_size_fc1():
    """FLUX fc1 (4608 x 3072 -> 12288, rank 32) in MXFP4: codes and scales
    of every row bit-exact, Y on sampled rows."""
    say("mx full-size fc1: building oracle case")
    case = C.named_case("fc1")
    pk = C.mx_pack(case)
    r = case["rank"]
    M, K = case["x"].shape
    N = pk["wq"].shape[0]
    layer = _mx_layer(case, pk)
    x = dev_bf16(case["x"])
    xq, xs, la = bq.quantize_act_lora_down(x, layer.smooth_inv, layer.lora_down, r, bq.MXFP4)
    y = bq.gemm_w4a4_lora_up(xq, xs, layer.wq, layer.ws, la, layer.lora_up, layer.bias, M, N, K, r, bq.MXFP4)
    torch.cuda.synchronize()
    ref_a = O.mx_quantize_act_lora_down(case["x"], pk["smooth_inv"], pk["l1"])
    assert np.array_equal(xq.cpu().numpy(), ref_a["xq"])
    assert np.array_equal(xs.cpu().numpy(), ref_a["xs"])
    t = ref_a["t"]
    assert np.allclose(la.cpu().numpy().astype(np.float64), t, rtol=1e-3, atol=1e-4 * np.max(np.abs(t)))
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, M - 1], rng.choice(M, 27, replace=False)]))
    ref = C.mx_oracle_rows(case, rows)
    sl = C.mx_slack(ref["xq"], ref["xs"], pk["wq"], pk["ws"], ref["t"], pk["l2"], case["bias"], t_from_kernel=True)
    assert_y_close(host_u16(y)[rows], ref["y"], "mx fc1 end to end", sl, ref["y64"])


def test_mx_full_size_fc2():
    """FLUX fc2 (4608 x 12288 -> 3072, rank 32, input bf16(GELU(fc1's Y)))
    in MXFP4: codes and scales of every row bit-exact, Y on sampled rows."""
    say("mx full-size fc2: building oracle case")
    case = C.mlp_pair()[1]
    pk = C.mx_pack(case)
    r = case["rank"]
    M, K = case["x"].shape
    N = pk["wq"].shape[0]
    say(f"mx full-size fc2: M={M} K={K} N={N} rank={r}")
    layer = _mx_layer(case, pk)
    x = dev_bf16(case["x"])
    xq, xs, la = bq.quantize_act_lora_down(x, layer.smooth_inv, layer.lora_down, r, bq.MXFP4)
    y = bq.gemm_w4a4_lora_up(xq, xs, layer.wq, layer.ws, la, layer.lora_up, layer.bias, M, N, K, r, bq.MXFP4)
    torch.cuda.synchronize()
    ref_a = O.mx_quantize_act_lora_down(case["x"], pk["smooth_inv"], pk["l1"])
    assert np.array_equal(xq.cpu().numpy(), ref_a["xq"])
    assert np.array_equal(xs.cpu().numpy(), ref_a["xs"])
    t = ref_a["t"]
    assert np.allclose(la.cpu().numpy().astype(np.float64), t, rtol=1e-3, atol=1e-4 * np.max(np.abs(t)))
    rng = np.random.default_rng(6)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, M - 1], rng.choice(M, 27, replace=False)]))
    ref = C.mx_oracle_rows(case, rows)
    sl = C.mx_slack(ref["xq"], ref["xs"], pk["wq"], pk["ws"], ref["t"], pk["l2"], case["bias"], t_from_kernel=True)
    assert_y_close(host_u16(y)[rows], ref["y"], "mx fc2 end to end", sl, ref["y64"])
