"""GPU parity of the fused MLP path (INT4): the first layer's GEMM kernel
with GELU fused (svdq_gemm_w4a4_lora_up_gelu) and with GELU plus the second
layer's kernel 1 fused (svdq_mlp_gemm_gelu_quant).

Bar: the GELU output within one bf16 unit of the oracle's GELU of the
kernel's own Y (fp32 vs fp64 evaluation: ~1 % of the outputs take the
neighbouring bf16 value); the fused codes and scales bit-exact against the oracle's
kernel 1 applied to that GELU output; lora_act2 within rtol 1e-3; the
pair's output within 1e-2 * max|Y| of the oracle run end to end."""

import numpy as np
import pytest
import torch

import bit_quantized_diffusion_amd as bq
import oracle as O
from tests import _cases as C
from tests.test_gpu_parity import assert_y_close, dev, dev_bf16, device_layer, host_u16, say

pytestmark = pytest.mark.gpu

# (M, K, N, rank, seed) of fc1 and (N2, rank2, seed2) of fc2; N % 128 == 0
PAIRS = [
    ((256, 512, 512, 16, 31), (256, 16, 32)),
    ((300, 576, 384, 32, 33), (200, 32, 34)),     # ragged M, odd group count in fc1
    ((129, 256, 128, 0, 35), (96, 48, 36)),       # fc1 rank 0, single N tile
    ((520, 1024, 640, 16, 37), (264, 0, 38)),     # fc2 rank 0
]


@pytest.fixture(autouse=True)
def _require_device():
    assert bq.device_check(0), "gfx950 device required for the GPU tests"


def _pair(p):
    (M, K, N, r, s), (N2, r2, s2) = p
    fc1 = C.small_case(M, K, N, r, s, True)
    fc2 = C.small_case(M, N, N2, r2, s2, True)
    return fc1, fc2


def _gelu_bits(y_bits):
    return O.f32_to_bf16_bits(O.gelu_tanh(O.bf16_bits_to_f32(y_bits)).astype(np.float32))


@pytest.mark.parametrize("p", PAIRS, ids=lambda p: "M%dK%dN%dr%d" % p[0][:4])
def test_gelu_epilogue(p):
    fc1, _ = _pair(p)
    say(f"gelu epilogue {p}")
    L1 = device_layer(fc1)
    M = fc1["x"].shape[0]
    x = dev_bf16(fc1["x"])
    xq, xs, la = bq.quantize_act_lora_down(x, L1.smooth_inv, L1.lora_down, L1.rank)
    y = bq.gemm_w4a4_lora_up(xq, xs, L1.wq, L1.ws, la, L1.lora_up, L1.bias, M, L1.N, L1.K, L1.rank)
    g = bq.gemm_w4a4_lora_up_gelu(xq, xs, L1.wq, L1.ws, la, L1.lora_up, L1.bias, M, L1.N, L1.K, L1.rank)
    torch.cuda.synchronize()
    yb, gb = host_u16(y), host_u16(g)
    want = _gelu_bits(yb)
    got64 = O.bf16_bits_to_f32(gb).astype(np.float64)
    want64 = O.bf16_bits_to_f32(want).astype(np.float64)
    # one bf16 unit, or 1e-30 absolute: near the fp32 underflow of
    # exp(-2u) the fp32 and fp64 tails part ways at values below 1e-30
    ulp = np.abs(want64) * 2.0 ** -7 + 1e-30
    assert np.all(np.abs(got64 - want64) <= ulp)
    # fp32 exp2 of an argument near |2u| carries a relative error of ~|u| *
    # 1e-7, so about 1 % of the outputs round to the neighbouring bf16 value
    say(f"  exact fraction {np.mean(gb == want):.5f}")
    assert np.mean(gb == want) > 0.98
    # and the layer + GELU against the oracle end to end
    ref = C.oracle_rows(fc1, np.arange(M))
    assert_y_close(gb, _gelu_bits(ref["y"]), "gelu layer")


@pytest.mark.parametrize("p", PAIRS, ids=lambda p: "M%dK%dN%dr%d" % p[0][:4])
def test_mlp_fused_pair(p):
    fc1, fc2 = _pair(p)
    say(f"mlp fused {p}")
    L1, L2 = device_layer(fc1), device_layer(fc2)
    M = fc1["x"].shape[0]
    x = dev_bf16(fc1["x"])
    xq, xs, la = bq.quantize_act_lora_down(x, L1.smooth_inv, L1.lora_down, L1.rank)
    xq2, xs2, la2 = bq.mlp_gemm_gelu_quant(xq, xs, L1.wq, L1.ws, la, L1.lora_up, L1.bias, M, L1.N, L1.K, L1.rank,
                                           L2.smooth_inv, L2.lora_down, L2.rank)
    g = bq.gemm_w4a4_lora_up_gelu(xq, xs, L1.wq, L1.ws, la, L1.lora_up, L1.bias, M, L1.N, L1.K, L1.rank)
    y2 = bq.gemm_w4a4_lora_up(xq2, xs2, L2.wq, L2.ws, la2, L2.lora_up, L2.bias, M, L2.N, L2.K, L2.rank)
    y2m = bq.mlp(x, L1, L2)
    torch.cuda.synchronize()
    # the fused quantizer = the oracle's kernel 1 on the same X2, bit for bit
    x2 = host_u16(g)
    pk2 = fc2["pk"]
    ref_a = O.quantize_act_lora_down(x2, pk2["smooth_inv"], pk2["l1"])
    assert np.array_equal(xq2.cpu().numpy(), ref_a["xq"])
    assert np.array_equal(host_u16(xs2), ref_a["xs"].view(np.uint16))
    if L2.rank:
        t = ref_a["t"]
        assert np.allclose(la2.cpu().numpy().astype(np.float64), t, rtol=1e-3, atol=1e-4 * np.max(np.abs(t)))
    # bq.mlp runs the same three kernels (lora_act2's atomic order may differ)
    assert_y_close(host_u16(y2m), host_u16(y2), "mlp() against the three calls")
    # the pair end to end against the oracle: fc1, GELU, fc2
    ref1 = C.oracle_rows(fc1, np.arange(M))
    ref2 = C.oracle_rows(fc2, np.arange(M), x_bits=_gelu_bits(ref1["y"]))
    assert_y_close(host_u16(y2), ref2["y"], "mlp pair")


def test_mlp_full_size_flux():
    """FLUX MLP pair at full size (fc1 4608x3072->12288, fc2 12288->3072,
    rank 32): fused codes and scales of every row bit-exact against the
    oracle's kernel 1 on the GELU output, the pair's output on sampled rows
    against the oracle end to end."""
    say("mlp full size: building oracle cases")
    fc1, fc2 = C.mlp_pair()
    L1, L2 = device_layer(fc1), device_layer(fc2)
    M = fc1["x"].shape[0]
    x = dev_bf16(fc1["x"])
    xq, xs, la = bq.quantize_act_lora_down(x, L1.smooth_inv, L1.lora_down, L1.rank)
    xq2, xs2, la2 = bq.mlp_gemm_gelu_quant(xq, xs, L1.wq, L1.ws, la, L1.lora_up, L1.bias, M, L1.N, L1.K, L1.rank,
                                           L2.smooth_inv, L2.lora_down, L2.rank)
    g = bq.gemm_w4a4_lora_up_gelu(xq, xs, L1.wq, L1.ws, la, L1.lora_up, L1.bias, M, L1.N, L1.K, L1.rank)
    y2 = bq.gemm_w4a4_lora_up(xq2, xs2, L2.wq, L2.ws, la2, L2.lora_up, L2.bias, M, L2.N, L2.K, L2.rank)
    torch.cuda.synchronize()
    rng = np.random.default_rng(9)
    rows = np.unique(np.concatenate([[0, 1, 4095, M - 1], rng.choice(M, 20, replace=False)]))
    x2 = host_u16(g)[rows]
    pk2 = fc2["pk"]
    ref_a = O.quantize_act_lora_down(x2, pk2["smooth_inv"], pk2["l1"])
    assert np.array_equal(xq2.cpu().numpy()[rows], ref_a["xq"])
    assert np.array_equal(host_u16(xs2)[:, rows], ref_a["xs"].view(np.uint16))
    t = ref_a["t"]
    assert np.allclose(la2.cpu().numpy()[rows].astype(np.float64), t, rtol=1e-3, atol=1e-4 * np.max(np.abs(t)))
    ref1 = C.oracle_rows(fc1, rows)
    ref2 = C.oracle_rows(fc2, np.arange(len(rows)), x_bits=_gelu_bits(ref1["y"]))
    assert_y_close(host_u16(y2)[rows], ref2["y"], "flux mlp pair")
