"""W4A16 comparison layer -- TEST INFRASTRUCTURE (same import rule as
``svdq_oracle``: only tests/, the smoke check and bench.py's cpu_baseline
leg use it; the HIP path never does).

The pages measure W4A4 against 4-bit weight-only models (W4A16): SVDQuant
abstract (3.0x over the W4A16 baseline with INT4, 3.1x with NVFP4) and the
blog's "Benchmarks".  They give no formula for that baseline.  Reading
(R14): the weights are quantized with the layer's own INT4 rule per output
channel in groups of 64 along K (no smoothing, no low-rank branch), the
activations stay bf16, each dequantized weight q * s (exact in fp32) is
rounded once to bf16, the operand type of a 16-bit matrix product, and
    Y = bf16(X . bf16(q s)^T + b)
with the product and the sum in fp64.
"""
from __future__ import annotations

import numpy as np

from .svdq_oracle import (bf16_bits_to_f32, f32_to_bf16_bits, quantize_groups, pack_int4, unpack_int4,
                          _bias64, GROUP)

__all__ = ["pack_w4a16", "w4a16_dequant", "w4a16_linear"]


def pack_w4a16(w_bits):
    """W bf16 [N][K] -> (wq uint8 [N][K/2], ws fp16 [K/64][N]): the INT4 rule
    on W itself, codes packed as the layer's other 4-bit codes."""
    w = bf16_bits_to_f32(np.asarray(w_bits, dtype=np.uint16))
    q, s = quantize_groups(w)
    return pack_int4(q), np.ascontiguousarray(s.T)


def w4a16_dequant(wq, ws, exact=False) -> np.ndarray:
    """Weights [N][K] from codes and group scales: bf16(q * s) as fp64, or
    q * s itself with exact=True."""
    q = unpack_int4(wq).astype(np.float64)
    s = np.asarray(ws).T.astype(np.float64)               # [N][K/64]
    w = q * np.repeat(s, GROUP, axis=1)                   # |q| <= 7, s fp16: exact
    if exact:
        return w
    return bf16_bits_to_f32(f32_to_bf16_bits(w.astype(np.float32))).astype(np.float64)


def w4a16_linear(x_bits, wq, ws, bias_bits=None):
    """Y = bf16(X . dequant(W)^T + b), fp64 inside."""
    x = bf16_bits_to_f32(np.asarray(x_bits, dtype=np.uint16)).astype(np.float64)
    w = w4a16_dequant(wq, ws)
    y64 = x @ w.T + _bias64(bias_bits, w.shape[0])[None, :]
    return dict(y=f32_to_bf16_bits(y64.astype(np.float32)), y64=y64)
