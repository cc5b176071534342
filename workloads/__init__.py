"""Seeded synthetic inputs for the ReLU-sparse gated FFN (TwELL) path.

This package only draws and lays out numbers: x, W_g^T, W_u^T and W_d for
each workload, on an exact-accumulation grid.  It computes nothing of the FFN
itself (no products, no activations, no packing).  Both the CPU oracle's tests
and the GPU path's tests / benchmark take their inputs from here.
"""

from .gen import (  # noqa: F401
    Workload,
    WORKLOADS,
    make_tiny,
    make_layer_0p5b,
    make_layer_2b,
    make_decode_windows,
    make_stress_layer,
    make_workload,
    make_random_small,
    bf16_representable,
    round_to_bf16,
)
