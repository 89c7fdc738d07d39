"""FLUX-shaped synthetic layer inputs (seeded, reproducible).

The pages measure whole FLUX.1 pipelines on trained weights with a calibration
dataset (model cards "svdq-int4-flux.1-dev", summary; SVDQuant abstract).
Neither weights nor data exist here, so layers of the same shapes are drawn:
tokens M = 4096 image + 512 text tokens for a 1024x1024 image, hidden size
3072, MLP width 12288, fused QKV width 9216.  Outliers are planted as a few
input channels whose activations (and matching weight input rows) are scaled
up, which is the situation the SVDQuant overview figure (stage 1) describes.

Every draw uses ``numpy.random.default_rng([config_id, stream_id])`` (PCG64):
stream 0 = X, 1 = W, 2 = bias, 3 = outlier channel set, 4 = LoRA A,
5 = LoRA B; the second layer of an MLP pair adds 10 to the stream id.
Samples are drawn in float32 and rounded to bfloat16 by torch's own
conversion (round to nearest even).
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch


# --------------------------------------------------------------------------
# dtype plumbing (library conversions, not the method)
# --------------------------------------------------------------------------

def f32_to_bf16_bits_torch(a: np.ndarray) -> np.ndarray:
    """float32 array -> bfloat16 bit patterns (uint16), torch's RNE cast."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32_torch(b: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(b, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(torch.float32).numpy()


# --------------------------------------------------------------------------
# layer specifications
# --------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class LayerSpec:
    name: str
    M: int
    K: int
    N: int
    rank: int
    config_id: int
    stream_base: int = 0          # +10 for the second layer of an MLP pair
    x_std: float = 1.0
    w_std: float = 0.02
    outlier_frac: float = 0.01
    x_outlier_scale: float = 20.0
    w_outlier_scale: float = 10.0
    bias_std: Optional[float] = None   # None -> no bias
    lora_rank: int = 0                 # extra LoRA adapter rank (merged)
    lora_std: float = 0.01
    x_from_prev: bool = False          # X is GELU(previous layer output)

    @property
    def n_outliers(self) -> int:
        return int(round(self.outlier_frac * self.K))


_FLUX_M = 4096 + 512     # 1024x1024 image tokens + text tokens
_FLUX_D = 3072
_FLUX_MLP = 4 * _FLUX_D

CONFIGS = {
    # tiny case, finishes in seconds on the CPU oracle
    "tiny": LayerSpec("tiny", 256, 512, 512, 16, config_id=0),
    # fused QKV projection of a FLUX block
    "qkv": LayerSpec("qkv", _FLUX_M, _FLUX_D, 3 * _FLUX_D, 32, config_id=1,
                     outlier_frac=0.005, x_outlier_scale=30.0,
                     w_outlier_scale=8.0, bias_std=0.01),
    # FLUX MLP pair: fc1 (3072 -> 12288) then fc2 (12288 -> 3072)
    "fc1": LayerSpec("fc1", _FLUX_M, _FLUX_D, _FLUX_MLP, 32, config_id=2,
                     outlier_frac=0.005, x_outlier_scale=30.0,
                     w_outlier_scale=8.0, bias_std=0.01),
    "fc2": LayerSpec("fc2", _FLUX_M, _FLUX_MLP, _FLUX_D, 32, config_id=2,
                     stream_base=10, outlier_frac=0.005, x_outlier_scale=1.0,
                     w_outlier_scale=8.0, bias_std=0.01, x_from_prev=True),
    # fc1 with an off-the-shelf rank-16 LoRA merged into the low-rank branch
    "fc1_lora": LayerSpec("fc1_lora", _FLUX_M, _FLUX_D, _FLUX_MLP, 32,
                          config_id=2, outlier_frac=0.005,
                          x_outlier_scale=30.0, w_outlier_scale=8.0,
                          bias_std=0.01, lora_rank=16),
}


def layer_spec(name: str, **overrides) -> LayerSpec:
    return dataclasses.replace(CONFIGS[name], **overrides)


def _rng(spec: LayerSpec, stream: int, config_id: Optional[int] = None):
    cid = spec.config_id if config_id is None else config_id
    return np.random.default_rng([cid, spec.stream_base + stream])


# --------------------------------------------------------------------------
# draws
# --------------------------------------------------------------------------

def gen_outlier_idx(spec: LayerSpec) -> np.ndarray:
    """Sorted set of outlier input channels (stream 3)."""
    n = spec.n_outliers
    if n == 0:
        return np.zeros(0, dtype=np.int64)
    idx = _rng(spec, 3).choice(spec.K, n, replace=False)
    return np.sort(idx).astype(np.int64)


def gen_x(spec: LayerSpec, idx: Optional[np.ndarray] = None) -> np.ndarray:
    """Activations X, bf16 bits [M][K]; outlier channels scaled up."""
    if idx is None:
        idx = gen_outlier_idx(spec)
    x = _rng(spec, 0).standard_normal((spec.M, spec.K), dtype=np.float32)
    x *= np.float32(spec.x_std)
    if len(idx):
        x[:, idx] *= np.float32(spec.x_outlier_scale)
    return f32_to_bf16_bits_torch(x)


def gen_w(spec: LayerSpec, idx: Optional[np.ndarray] = None) -> np.ndarray:
    """Weights in nn.Linear layout, bf16 bits [N][K]; the input rows that
    meet the outlier channels are scaled up."""
    if idx is None:
        idx = gen_outlier_idx(spec)
    w = _rng(spec, 1).standard_normal((spec.N, spec.K), dtype=np.float32)
    w *= np.float32(spec.w_std)
    if len(idx):
        w[:, idx] *= np.float32(spec.w_outlier_scale)
    return f32_to_bf16_bits_torch(w)


def gen_bias(spec: LayerSpec) -> Optional[np.ndarray]:
    if spec.bias_std is None:
        return None
    b = _rng(spec, 2).standard_normal(spec.N, dtype=np.float32)
    b *= np.float32(spec.bias_std)
    return f32_to_bf16_bits_torch(b)


def gen_lora(spec: LayerSpec):
    """Off-the-shelf LoRA adapter (A [K][ra], B [ra][N]) in bf16 bits, drawn
    from the LoRA layer's own config id streams 4 and 5."""
    ra = spec.lora_rank
    if ra == 0:
        return None, None
    cid = spec.config_id + 1
    a = _rng(spec, 4, cid).standard_normal((spec.K, ra), dtype=np.float32)
    b = _rng(spec, 5, cid).standard_normal((ra, spec.N), dtype=np.float32)
    a *= np.float32(spec.lora_std)
    b *= np.float32(spec.lora_std)
    return f32_to_bf16_bits_torch(a), f32_to_bf16_bits_torch(b)


def gen_layer(spec: LayerSpec):
    """X (unless it comes from the previous layer), W, bias, outlier set."""
    idx = gen_outlier_idx(spec)
    x = None if spec.x_from_prev else gen_x(spec, idx)
    return dict(x=x, w=gen_w(spec, idx), bias=gen_bias(spec), outliers=idx)


def custom_spec(M: int, K: int, N: int, rank: int, seed: int,
                bias: bool = True, **kw) -> LayerSpec:
    """Small test-sized layers with the tiny config's distributions."""
    return LayerSpec(f"custom{M}x{K}x{N}r{rank}s{seed}", M, K, N, rank,
                     config_id=1000 + seed,
                     bias_std=0.01 if bias else None, **kw)
