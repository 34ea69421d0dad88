"""MI355X (gfx950) sparse Mixture-of-Experts FFN layer: FP8 block-scaled grouped GEMMs.

The compute runs in hand-written HIP kernels inside ``libmoe_mi355x.so`` (C ABI in
include/moe.h); this package is its Python binding.  Build with
``python -m sparse_moe_ffn_gemm_amd.build``.
"""
from ._lib import (PROFILE_STAGES, MoEError, Routing, WorkspaceRegions, forward, forward_profiled, lib, new_routing, new_workspace,
                   quantize_activations, quantize_weights, route, workspace_bytes, workspace_layout)
from .layer import MoELayer

__all__ = ["PROFILE_STAGES", "MoEError", "Routing", "WorkspaceRegions", "forward", "forward_profiled", "lib", "new_routing",
           "new_workspace", "quantize_activations", "quantize_weights", "route",
           "workspace_bytes", "workspace_layout", "MoELayer"]
