"""Block-scaled FP4 routed-expert MoE layer and 4/6 quantizer for MI355X (gfx950).

The computation lives in hand-written HIP kernels behind the C ABI of
include/fp4moe.h (libfp4moe.so, built by `python -m
block_scaled_fp4_nvfp4_amd.build`).  This package is its thin Python binding.
"""
from ._lib import (FMT, RULE, STAGES, Fp4Error, MoELayer, StageTimer, block_error, dequantize,
                   lib, moe_forward, moe_forward_noalloc, moe_forward_profiled, quantize, quantize_hessian, route, status_string,
                   tile_weights, workspace_layout, workspace_size)

__all__ = ["FMT", "RULE", "STAGES", "Fp4Error", "MoELayer", "StageTimer", "block_error", "dequantize",
           "lib", "moe_forward", "moe_forward_noalloc", "moe_forward_profiled", "quantize", "quantize_hessian", "route", "status_string",
           "tile_weights", "workspace_layout", "workspace_size"]
