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


def mx_pack(case):
    """MXFP4 weights of a case: the same smoothing and SVD branch, the
    residual quantized in MXFP4 by the oracle."""
    return O.mx_pack_weights(None, None, case["rank"], svd_cache=case["pk"])


def mx_oracle_rows(case, rows, x_bits=None):
    """MXFP4 oracle of the whole layer on a subset of token rows."""
    x = case["x"] if x_bits is None else x_bits
    pk = mx_pack(case)
    sub = np.ascontiguousarray(x[rows])
    a = O.mx_quantize_act_lora_down(sub, pk["smooth_inv"], pk["l1"])
    b = O.mx_gemm_lora_up(a["xq"], a["xs"], pk["wq"], pk["ws"], a["t"], pk["l2"], case["bias"])
    b.update(a)
    return b
