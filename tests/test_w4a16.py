"""W4A16 comparison layer (4-bit weights, bf16 activations) on the CPU:
the W4A16 oracle pinned against exact rational arithmetic and the grid
cases where it must be lossless, and the library's host pack against it
bit for bit."""

from fractions import Fraction

import numpy as np
import pytest

import bit_quantized_diffusion_amd as bq
import oracle as O
from tests.test_oracle import round_to_format


def _bf16(a):
    return O.f32_to_bf16_bits(np.asarray(a, np.float32))


def _grid_weights(rng, N, K):
    """W = q * 2^e with q in [-7, 7], a 7 in every group of 64: the group's
    scale is exactly 2^e, every weight is a bf16 value and round trips."""
    q = rng.integers(-7, 8, size=(N, K))
    q[:, ::64] = 7 * rng.choice([-1, 1], size=(N, K // 64))
    e = rng.integers(-12, 4, size=(N, K // 64))
    w = q * np.exp2(np.repeat(e, 64, axis=1))
    return q, e, w


def test_grid_weights_are_lossless():
    rng = np.random.default_rng(61)
    q, e, w = _grid_weights(rng, 24, 256)
    wq, ws = O.pack_w4a16(_bf16(w))
    assert ws.shape == (4, 24) and ws.dtype == np.float16
    assert np.array_equal(ws.T.astype(np.float64), np.exp2(e))
    assert np.array_equal(O.unpack_int4(wq), q)
    assert np.array_equal(O.w4a16_dequant(wq, ws), w)


def test_linear_matches_exact_rational_sum():
    """Y on a tiny case against sums of Fractions: y64 within fp64 rounding
    of the exact X . bf16(q s)^T + b, y its bf16 rounding."""
    rng = np.random.default_rng(62)
    M, K, N = 3, 128, 5
    x = _bf16(rng.standard_normal((M, K)))
    w = _bf16(rng.standard_normal((N, K)) * 0.3)
    b = _bf16(rng.standard_normal(N))
    wq, ws = O.pack_w4a16(w)
    out = O.w4a16_linear(x, wq, ws, b)
    xf = O.bf16_bits_to_f32(x).astype(np.float64)
    bf = O.bf16_bits_to_f32(b).astype(np.float64)
    codes = O.unpack_int4(wq)
    for n in range(N):
        wrow = []
        for k in range(K):
            # dequantize one weight: code times its group's fp16 scale, then
            # the nearest bf16 (8 significant bits, ties to even)
            exact = int(codes[n, k]) * Fraction(float(ws[k // 64, n]))
            wrow.append(round_to_format(exact, 8, -126))
        for m in range(M):
            y = sum(Fraction(float(xf[m, k])) * wrow[k] for k in range(K)) + Fraction(float(bf[n]))
            assert abs(Fraction(float(out["y64"][m, n])) - y) <= abs(y) * Fraction(1, 2 ** 45) + Fraction(1, 2 ** 1000)
            assert out["y"][m, n] == _bf16(float(out["y64"][m, n]))


def test_dequant_rounds_to_bf16_once():
    """An fp16 scale with more than 8 significant bits makes q * s fall
    between bf16 values: dequant is the nearest one (ties to even), and the
    exact form keeps q * s."""
    s = np.float16(1.0 + 2.0 ** -10)                  # 11 significant bits
    q = np.array([[7, -7, 3, 1, 0, -5] + [0] * 58], dtype=np.int8)
    wq = O.pack_int4(q)
    ws = np.array([[s]], dtype=np.float16)
    exact = O.w4a16_dequant(wq, ws, exact=True)[0, :6]
    assert np.array_equal(exact, q[0, :6] * float(s))
    got = O.w4a16_dequant(wq, ws)[0, :6]
    for v, g in zip(exact, got):
        assert Fraction(float(g)) == round_to_format(Fraction(float(v)), 8, -126)
    assert got[0] != exact[0]                         # 7 * (1 + 2^-10) is not a bf16 value


def test_error_bound_against_weights():
    """|bf16(q s) - w| <= s / 2 + 2^-8 |q s| for every weight: half a step of
    the group's grid plus one bf16 rounding (unit roundoff 2^-8)."""
    rng = np.random.default_rng(63)
    w = _bf16(rng.standard_normal((40, 512)) * np.exp2(rng.integers(-6, 6, size=(40, 1))))
    wq, ws = O.pack_w4a16(w)
    wf = O.bf16_bits_to_f32(w).astype(np.float64)
    d = O.w4a16_dequant(wq, ws)
    s = np.repeat(ws.T.astype(np.float64), 64, axis=1)
    assert np.all(np.abs(d - wf) <= s / 2 * (1 + 2.0 ** -10) + 2.0 ** -8 * np.abs(d))


def test_zero_group_and_bias():
    w = np.zeros((2, 128), np.float32)
    w[1, 64:] = 1.5
    wq, ws = O.pack_w4a16(_bf16(w))
    assert float(ws[0, 0]) == 0 and float(ws[0, 1]) == 0
    x = _bf16(np.ones((1, 128)))
    out = O.w4a16_linear(x, wq, ws, _bf16([0.25, -2.0]))
    assert out["y64"][0, 0] == 0.25
    assert out["y64"][0, 1] == 64 * 1.5 - 2.0


@pytest.mark.parametrize("N,K,seed", [(8, 64, 1), (200, 448, 2), (131, 1024, 3)])
def test_host_pack_bit_exact(N, K, seed):
    rng = np.random.default_rng(seed)
    w = _bf16(rng.standard_normal((N, K)) * np.exp2(rng.integers(-8, 8, size=(N, 1))))
    w[0, :64] = 0                                      # an all-zero group
    wq, ws = bq.pack_w4a16(w)
    rq, rs = O.pack_w4a16(w)
    assert np.array_equal(wq, rq)
    assert np.array_equal(ws.view(np.uint16), rs.view(np.uint16))
