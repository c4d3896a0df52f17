"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This package only draws and encodes inputs (random normals, bf16 and fp8
encodings, block scales).  It holds none of the layer's arithmetic: no
routing, no expert projection, no normalisation.
"""

from .layer_inputs import (  # noqa: F401
    LayerShape,
    LayerInputs,
    WORKLOADS,
    WORKLOAD_ORDER,
    make_layer,
    make_layer_from_arrays,
    quantize_blocks,
    f32_to_bf16_bits,
    tokens_subset,
)
