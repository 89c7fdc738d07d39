"""Case builders shared by the GPU tests: inputs from ``synth``, packed
weights and expected values from the oracle.  Nothing here takes a value
from the HIP path."""

from __future__ import annotations

import functools

import numpy as np

import oracle as O
import synth


def absmax_cols(x_bits) -> np.ndarray:
    return np.abs(O.bf16_bits_to_f32(x_bits)).max(axis=0).astype(np.float32)


@functools.lru_cache(maxsize=None)
def small_case(M, K, N, rank, seed, bias=True, lora_rank=0):
    spec = synth.custom_spec(M, K, N, rank, seed=seed, bias=bias, lora_rank=lora_rank)
    return _build(spec)


@functools.lru_cache(maxsize=None)
def named_case(name):
    spec = synth.layer_spec(name)
    return _build(spec)


def _build(spec):
    lay = synth.gen_layer(spec)
    ax = absmax_cols(lay["x"])
    pk = O.pack_weights(lay["w"], ax, spec.rank)
    if spec.lora_rank:
        a_bits, b_bits = synth.gen_lora(spec)
        l1, l2 = O.merge_lora(pk["l1"], pk["l2"], pk["smooth_inv"], a_bits, b_bits)
        pk = dict(pk, l1=l1, l2=l2)
    rank = pk["l1"].shape[1]
    pk.pop("w_hat", None)
    return dict(spec=spec, x=lay["x"], w=lay["w"], bias=lay["bias"], ax=ax, pk=pk, rank=rank)


def oracle_rows(case, rows, x_bits=None):
    """Oracle of the whole layer on a subset of token rows (every step is
    row-local in M, so this equals the full oracle restricted to `rows`)."""
    x = case["x"] if x_bits is None else x_bits
    pk = case["pk"]
    sub = np.ascontiguousarray(x[rows])
    a = O.quantize_act_lora_down(sub, pk["smooth_inv"], pk["l1"])
    b = O.gemm_w4a4_lora_up(a["xq"], a["xs"], pk["wq"], pk["ws"], a["t"], pk["l2"], case["bias"])
    b.update(a)
    return b


@functools.lru_cache(maxsize=None)
def mlp_pair():
    """FLUX MLP pair: fc1 (oracle-packed) and fc2 whose input is
    bf16(GELU_tanh(Y_fc1)) with Y_fc1 the oracle's fc1 output."""
    fc1 = named_case("fc1")
    y1 = O.svdq_linear(fc1["x"], fc1["pk"], fc1["bias"], per_group=False)["y"]
    x2 = O.f32_to_bf16_bits(O.gelu_tanh(O.bf16_bits_to_f32(y1)).astype(np.float32))
    spec2 = synth.layer_spec("fc2")
    ax2 = absmax_cols(x2)
    idx = np.sort(np.argsort(-ax2, kind="stable")[: spec2.n_outliers])
    w2 = synth.gen_w(spec2, idx)
    b2 = synth.gen_bias(spec2)
    pk2 = O.pack_weights(w2, ax2, spec2.rank)
    pk2.pop("w_hat", None)
    fc2 = dict(spec=spec2, x=x2, w=w2, bias=b2, ax=ax2, pk=pk2, rank=spec2.rank)
    return fc1, fc2


_MX_PACKS = {}


def mx_pack(case):
    """MXFP4 weights of a case: the same smoothing and SVD branch, the
    residual quantized in MXFP4 by the oracle.  Computed once per case and
    shared between tests, which only read it."""
    key = id(case["pk"])
    hit = _MX_PACKS.get(key)
    if hit is None or hit[0] is not case["pk"]:
        pk = O.mx_pack_weights(None, None, case["rank"], svd_cache=case["pk"])
        hit = _MX_PACKS[key] = (case["pk"], pk)
    return hit[1]


def mx_oracle_rows(case, rows, x_bits=None):
    """MXFP4 oracle of the whole layer on a subset of token rows."""
    x = case["x"] if x_bits is None else x_bits
    pk = mx_pack(case)
    sub = np.ascontiguousarray(x[rows])
    a = O.mx_quantize_act_lora_down(sub, pk["smooth_inv"], pk["l1"])
    b = O.mx_gemm_lora_up(a["xq"], a["xs"], pk["wq"], pk["ws"], a["t"], pk["l2"], case["bias"])
    b.update(a)
    return b


# ---------------------------------------------------------------------------
# per-element output bounds (from the oracle's own terms, never from the GPU)
# ---------------------------------------------------------------------------

def ulp_bf16(v) -> np.ndarray:
    """Spacing of bf16 values at |v| (bf16 keeps 8 significant bits; below
    2^-126 the spacing is that of the subnormals, 2^-133)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(np.where(a > 0, e, -126), -126)
    return np.exp2(e - 7)


def int4_slack(ref, xs, ws, t, l2_bits, bias_bits, t_from_kernel):
    """Per-element slack of the fp32 pre-rounding sum against the oracle's
    exact one, for an INT4 layer whose oracle terms are in `ref`
    (gemm_w4a4_lora_up's P).

    The GPU adds the G dequantized group partials with one fp32 FMA each,
    the rank-r up projection with fp32 matrix-core accumulation and the
    bias, so its sum differs from the exact one by at most about
    (G + r + 2) fp32 roundings of the running magnitude; twice that is used.
    When lora_act comes from the GPU's kernel 1 (a different summation order
    than the oracle's fp64), bf16(t) can land one bf16 step away: one
    ulp_bf16(t_j) |L2_jn| per rank component is allowed for it."""
    P = np.abs(np.asarray(ref["P"], dtype=np.float64))          # [M][N][G]
    sx = np.asarray(xs).astype(np.float64)                      # [G][M]
    sw = np.asarray(ws).astype(np.float64)                      # [G][N]
    A = np.einsum("mng,gm,gn->mn", P, sx, sw)
    G = P.shape[2]
    l2 = O.bf16_bits_to_f32(l2_bits).astype(np.float64)
    r = l2.shape[0]
    U = np.zeros_like(A)
    T = np.zeros_like(A)
    if r:
        tb = O.bf16_bits_to_f32(O.f32_to_bf16_bits(np.asarray(t).astype(np.float32))).astype(np.float64)
        U = np.abs(tb) @ np.abs(l2)
        if t_from_kernel:
            T = ulp_bf16(np.asarray(t, np.float64)) @ np.abs(l2)
    B = np.zeros(A.shape[1]) if bias_bits is None else np.abs(O.bf16_bits_to_f32(bias_bits).astype(np.float64))
    gamma = 2.0 * (G + r + 2) * 2.0 ** -24
    return gamma * (A + U + B[None, :]) + T


def mx_slack(ref_a_xq, ref_a_xs, wq, ws, t, l2_bits, bias_bits, t_from_kernel):
    """As int4_slack for the MXFP4 layer: the decoded operands' |a||b| sum
    replaces the per-group partials; the matrix core accumulates K/64
    instructions' results in fp32."""
    a = np.abs(O.mx_decode(O.mxfp4_oracle._unpack_nibbles(ref_a_xq), np.asarray(ref_a_xs).T))
    b = np.abs(O.mx_decode(O.mxfp4_oracle._unpack_nibbles(wq), np.asarray(ws).T))
    A = a @ b.T
    K = a.shape[1]
    l2 = O.bf16_bits_to_f32(l2_bits).astype(np.float64)
    r = l2.shape[0]
    U = np.zeros_like(A)
    T = np.zeros_like(A)
    if r:
        tb = O.bf16_bits_to_f32(O.f32_to_bf16_bits(np.asarray(t).astype(np.float32))).astype(np.float64)
        U = np.abs(tb) @ np.abs(l2)
        if t_from_kernel:
            T = ulp_bf16(np.asarray(t, np.float64)) @ np.abs(l2)
    B = np.zeros(A.shape[1]) if bias_bits is None else np.abs(O.bf16_bits_to_f32(bias_bits).astype(np.float64))
    gamma = 2.0 * (K // 64 + r + 2) * 2.0 ** -24
    return gamma * (A + U + B[None, :]) + T
