"""Seeded synthetic inputs for the HelixLinear forward pass.

This package is the input side shared by the tests, the bench and the smoke
check.  It plays the role of the offline HXQ codec described in the HXQ
whitepaper (Fellows, Echo Labs, 2026), "Method" (per-tensor k-means, index
assignment, sidecar outlier correction, 12-bit index packing) and "2D vector
quantization": it draws weights, fits the codebooks, assigns indices, picks the
sidecar and writes the packed bytes.  It computes no part of the forward pass:
no dequantised product, no sidecar applied to activations, no bias add.
"""

from .gen import (  # noqa: F401
    CONFIGS,
    Layer,
    config_layers,
    pack12_rows,
    random_layer,
    synth_layer,
    synth_x,
    to_bf16_bits,
)
