"""MI355X (gfx950) sparse Mixture-of-Experts FFN layer: FP8 grouped GEMMs with 128x128
block-scaled or MXFP8 (1x32, E8M0) weights.

The compute runs in hand-written HIP kernels inside ``libmoe_mi355x.so`` (C ABI in
include/moe.h); this package is its Python binding.  Build with
``python -m sparse_moe_ffn_gemm_amd.build``.
"""
from ._lib import (PROFILE_STAGES, MoEError, Routing, WorkspaceRegions, forward, forward_fused,
                   forward_profiled, fused_status, lib, mx_row,
                   new_routing, new_workspace, quantize_activations, quantize_activations_mx,
                   quantize_weights, quantize_weights_mx, quantize_weights_mxfp4, mxfp4_shapes, mx_scale_shape,
                   route,
                   workspace_bytes, workspace_layout)
from .layer import MoELayer

__all__ = ["PROFILE_STAGES", "MoEError", "Routing", "WorkspaceRegions", "forward", "forward_fused",
           "forward_profiled", "fused_status", "lib", "new_routing",
           "new_workspace", "quantize_activations", "quantize_activations_mx", "quantize_weights",
           "quantize_weights_mx", "quantize_weights_mxfp4", "mxfp4_shapes", "mx_scale_shape", "mx_row", "route",
           "workspace_bytes", "workspace_layout", "MoELayer"]
