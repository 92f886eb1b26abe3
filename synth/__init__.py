"""Seeded synthetic inputs for the routed-MoE block.

This package draws the block's inputs (activations, weights, the residual
stream) from numpy's PCG64 generator in a fixed order.  It holds none of the
block's arithmetic: the only operations here are random draws, the
round-to-nearest-even conversion of drawn fp32 values to bf16 storage, and the
packing of drawn E2M1 codes two to a byte.  Both the CPU oracle and the GPU
path take their inputs from here.
"""

from .inputs import (  # noqa: F401
    CONFIGS,
    BlockInputs,
    Dims,
    f32_to_bf16_bits,
    bf16_bits_to_f32,
    make_attn_side,
    make_block,
    make_c3_block,
    make_c4_layer,
    make_c4_stream,
    hot_experts,
    skew_delta,
    routing_inputs,
)
