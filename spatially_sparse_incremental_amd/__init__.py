"""Tile-sparse incremental convolution (SIGE hot path) for AMD MI355X (gfx950).

The compute lives in libsige.so (HIP kernels behind the C ABI of
include/sige.h); this package is the ctypes binding over it.
"""
from ._lib import (  # noqa: F401
    DTYPE_CODE,
    EXPORTS,
    Derived,
    Geom,
    LayerPlan,
    SigeError,
    geom,
    lib,
    sige_conv_blocks,
    sige_diff_mask,
    sige_diff_mask_bits,
    sige_gather,
    sige_geom_derive,
    sige_max_blocks,
    sige_reduce_bits,
    sige_reduce_bits_copy,
    sige_reduce_bits_layers,
    sige_reduce_mask,
    sige_reduce_mask_copy,
    sige_restore_blocks,
    sige_scatter,
    sige_sparse_attention,
    sige_sparse_attention_workspace,
    sige_sparse_conv_layer,
    sige_sparse_conv_layer_auto,
    sige_sparse_conv_layer_plan,
    sige_sparse_conv_layer_restore,
    sige_noalloc_scratch_bytes,
    sige_sparse_conv_layer_split,
    sige_sparse_conv_layer_split_noalloc,
    sige_sparse_conv_layer_split_workspace,
    weight_to_krsc,
)
