"""MXFP4 variant of the oracle -- TEST INFRASTRUCTURE (same import rule as
``svdq_oracle``).

The pages quantize to NVFP4 on Blackwell ("Native loading in Diffusers":
precision nvfp4, group_size 16; SVDQuant abstract: NVFP4 on the RTX 5090).
That scale format is NVIDIA's.  Its CDNA4 counterpart is OCP Microscaling
MXFP4: FP4 E2M1 elements with one E8M0 power-of-two scale per 32-element
block along K.  The rules below follow the OCP MX v1.0 definition:

  M1  block = 32 consecutive k of one row.
  M2  amax = max |v| over the block (fp32).  amax == 0 -> scale byte 0 and
      all codes 0.  Otherwise e = clamp(floor(log2 amax) - 2, -127, 127),
      floor(log2) read from the fp32 exponent field (subnormals give -127),
      scale byte = e + 127, scale = 2^e.  (2 = exponent of E2M1's largest
      value 6 = 1.5 * 2^2.)
  M3  element code = v / 2^e rounded to the E2M1 grid
      {0, 0.5, 1, 1.5, 2, 3, 4, 6}, ties to the even code, magnitudes above
      6 saturate to 6.  The sign bit is set only for a non-zero magnitude
      (a value that rounds to zero is stored as +0).
  M4  packing: low nibble = even k; scales group-major [K/32][rows].
  M5  decode is exact: value = sign * grid[code & 7] * 2^(byte - 127).
      The GEMM is the fp64 product of the decoded operands.

Smoothing, the SVD branch and the output rounding are the INT4 oracle's.
"""

from __future__ import annotations

import numpy as np

from .svdq_oracle import (bf16_bits_to_f32, f32_to_bf16_bits, smooth_act,
                          lora_up, _bias64)

__all__ = [
    "MX_BLOCK", "E2M1_GRID", "mx_quantize_blocks", "mx_decode",
    "mx_pack_weights", "mx_quantize_act_lora_down", "mx_gemm_lora_up",
    "e2m1_round_code",
]

MX_BLOCK = 32
E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_round_code(a) -> np.ndarray:
    """Non-negative magnitudes (fp64, already divided by the block scale) ->
    3-bit E2M1 magnitude code, nearest grid value, ties to the even code."""
    a = np.asarray(a, dtype=np.float64)
    d = np.abs(a[..., None] - E2M1_GRID)          # distance to each grid point
    best = d.min(axis=-1, keepdims=True)
    cand = d == best                               # one or two candidates
    idx = np.arange(8)
    # among tied candidates prefer the even code
    score = np.where(cand, np.where(idx % 2 == 0, 0, 1) * 16 + idx, 1000)
    code = score.argmin(axis=-1)
    code = np.where(a >= 6.0, 7, code)
    return code.astype(np.uint8)


def _floor_log2_f32(amax):
    bits = np.asarray(amax, dtype=np.float32).view(np.uint32)
    expo = ((bits >> 23) & 0xFF).astype(np.int64)
    return expo - 127                              # fp32 subnormals -> -127


def mx_quantize_blocks(v):
    """fp32 rows [rows][K] (K % 32 == 0) -> (codes uint8 [rows][K] with the
    sign in bit 3, scale bytes uint8 [rows][K/32])."""
    v = np.asarray(v, dtype=np.float32)
    rows, K = v.shape
    assert K % MX_BLOCK == 0
    b = v.reshape(rows, K // MX_BLOCK, MX_BLOCK)
    amax = np.abs(b).max(axis=2)
    e = np.clip(_floor_log2_f32(amax) - 2, -127, 127)
    zero = amax == 0
    e = np.where(zero, -127, e)
    scaled = b.astype(np.float64) * np.exp2(-e.astype(np.float64))[:, :, None]
    mag = e2m1_round_code(np.abs(scaled))
    sign = ((scaled < 0) & (mag > 0)).astype(np.uint8)
    codes = (mag | (sign << 3)).astype(np.uint8)
    codes[zero] = 0
    return codes.reshape(rows, K), (e + 127).astype(np.uint8)


def mx_decode(codes, scale_bytes) -> np.ndarray:
    """codes uint8 [rows][K] (unpacked nibbles), scale bytes [rows][K/32]
    -> exact fp64 values."""
    codes = np.asarray(codes, dtype=np.uint8)
    mag = E2M1_GRID[codes & 7]
    sgn = np.where(codes & 8, -1.0, 1.0)
    sc = np.exp2(np.asarray(scale_bytes, dtype=np.float64) - 127.0)
    return sgn * mag * np.repeat(sc, MX_BLOCK, axis=1)


def _pack_nibbles(codes):
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def _unpack_nibbles(p):
    p = np.asarray(p, dtype=np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    return out


def mx_pack_weights(w_bits, act_absmax, rank, svd_cache=None):
    """Offline pack for MXFP4: smoothing and SVD as INT4, residual in MXFP4.
    Returns smooth_inv, l1, l2, wq uint8 [N][K/2], ws uint8 [K/32][N], r."""
    from .svdq_oracle import pack_weights
    base = svd_cache if svd_cache is not None else pack_weights(w_bits, act_absmax, rank)
    codes, sb = mx_quantize_blocks(np.ascontiguousarray(base["r"].T))
    out = dict(base)
    out.update(wq=_pack_nibbles(codes), ws=np.ascontiguousarray(sb.T))
    return out


def mx_quantize_act_lora_down(x_bits, smooth_inv, l1_bits):
    xh_bits = smooth_act(x_bits, smooth_inv)
    xh = bf16_bits_to_f32(xh_bits)
    codes, sb = mx_quantize_blocks(xh)
    l1 = bf16_bits_to_f32(l1_bits).astype(np.float64)
    t = xh.astype(np.float64) @ l1 if l1.shape[1] else np.zeros((xh.shape[0], 0))
    return dict(xhat=xh_bits, xq=_pack_nibbles(codes),
                xs=np.ascontiguousarray(sb.T), t=t)


def mx_gemm_lora_up(xq, xs, wq, ws, t, l2_bits, bias_bits=None):
    a = mx_decode(_unpack_nibbles(xq), np.asarray(xs).T)
    b = mx_decode(_unpack_nibbles(wq), np.asarray(ws).T)
    acc = a @ b.T
    up = lora_up(t, l2_bits)
    y64 = acc + up + _bias64(bias_bits, acc.shape[1])[None, :]
    return dict(y=f32_to_bf16_bits(y64.astype(np.float32)), y64=y64, acc=acc, up=up)

