"""Seeded synthetic inputs for the fused MoE layer.

This package holds only input generation: random draws, the dtype
conversions that put the draws into storage form, and the shapes of the
workloads.  It contains none of the layer's arithmetic (no routing, no
sorting, no expert contraction, no combine), so that the HIP path and the
oracle can both consume it without sharing any computation.
"""
from .gen import (  # noqa: F401
    CONFIGS,
    LayerConfig,
    counter_normal,
    layer_batch,
    layer_weights,
    normal_bf16,
    normal_f32,
    quant_int4_groups,
)
