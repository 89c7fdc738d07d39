"""Seeded synthetic inputs for the SVDQuant W4A4 linear layer.

This module only draws random numbers and rounds them to the storage dtype.
It holds none of the method's arithmetic (no smoothing, no SVD, no
quantization), so both the CPU oracle and the GPU path can take their inputs
from it without sharing any code of the method.
"""

from .flux_layers import (  # noqa: F401
    LayerSpec,
    CONFIGS,
    layer_spec,
    gen_x,
    gen_w,
    gen_bias,
    gen_outlier_idx,
    gen_lora,
    gen_layer,
    custom_spec,
    f32_to_bf16_bits_torch,
    bf16_bits_to_f32_torch,
)
