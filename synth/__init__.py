"""Seeded synthetic inputs for the DeepSeekMoE layer forward.

This package only draws random numbers and rounds them to the storage type.
It holds none of the layer's arithmetic (no logits, no softmax, no FFN), so
both the fp64 oracle and the HIP path can take their inputs from it without
sharing any of the method's code.
"""
from .configs import CONFIGS, LayerConfig, get_config  # noqa: F401
from .generate import (  # noqa: F401
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    make_inputs,
    redraw_x_rows,
    zipf_bias,
)
