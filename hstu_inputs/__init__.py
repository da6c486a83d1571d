"""Seeded synthetic inputs for the HSTU jagged layer forward.

This package only draws random numbers and arranges them in the layouts the
layer consumes (jagged offsets, timestamps, weights, bias tables, embedding
ids). It performs none of the layer's arithmetic, so both the CPU oracle and
the GPU path can take their inputs from it without sharing any of the method.
"""

from .gen import (  # noqa: F401
    CONFIG_NAMES,
    LayerParams,
    Workload,
    bf16_bits,
    bf16_round,
    make_config,
    make_jagged,
    make_layer_params,
    make_timestamps,
)
