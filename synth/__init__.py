"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the bench.

This package only draws random numbers and rasterises edit shapes.  It holds
none of the sparse-inference arithmetic (no diff, pooling, block selection or
convolution), so both sides of a parity test can take their inputs from it.
"""
from .gen import (  # noqa: F401
    DTYPES,
    Blob,
    LayerSpec,
    SWEEP,
    StarPolygon,
    Workload,
    WORKLOADS,
    blob_mask,
    edit_shape,
    make_activation,
    make_edit,
    make_layer_tensors,
    polygon_mask,
    rectangle_mask,
    workload,
)
