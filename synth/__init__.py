"""Seeded synthetic inputs for the top-k MoE layer forward.

This package draws input tensors and nothing else: it holds none of the layer's
arithmetic (no router, no softmax, no top-k, no dispatch, no experts). Both the
CPU oracle's tests and the GPU path's tests and benchmark take their inputs from
here, so that the two sides see bit-identical values.
"""

from .inputs import (  # noqa: F401
    CONFIGS,
    LayerSpec,
    LayerInputs,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    make_inputs,
    RouterNoise,
    make_router_noise,
    spec,
)
