"""Seeded synthetic inputs for the Stable LatentMoE layer.

This module is the only code shared by the CPU oracle and the GPU path. It
holds the five layer configurations (shapes, dtypes, seeds and input
recipes) and one counter-based generator (``synth_core.h``), compiled for the
host and for the device. It contains none of the layer's arithmetic.
"""
from .configs import CONFIGS, LayerConfig, TENSOR_IDS, tensor_spec, tensor_names  # noqa: F401
from .gen import (  # noqa: F401
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    host_tensor,
    host_inputs,
    to_f64,
)
