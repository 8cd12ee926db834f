"""Routed-expert FP8 block-scaled MoE decode for MI355X (gfx950).

The compute path is the HIP library libmoe_decode.so (C ABI in
include/moe_decode.h and include/moe_boundary.h); this package is its thin
Python binding. Build the
library with `python -m fp8_block_scaled_moe_amd.build`.
"""

from ._capi import (  # noqa: F401
    MoeDecode,
    MoeDecodeConfig,
    MoeDecodeError,
    debug_codec,
    debug_codec_fp4,
    error_string,
    header_functions,
    lib,
    mxfp8_quantize,
    reduce_rmsnorm,
)
