"""One GPU's routed-expert (mixture-of-experts) layer for AMD MI355X (gfx950).

The compute path is the HIP library libtre_moe.so (C ABI in include/moe.h);
this package only marshals torch tensors into its calls.
"""
from . import _native
from .ops import (MoeError, make_shape, moe_grouped_gemm_bwd, moe_grouped_gemm_fwd,
                  moe_layer_bwd, moe_layer_fwd, moe_permute, moe_route, moe_status_str,
                  moe_unpermute, moe_workspace_bytes)

__all__ = ["MoeError", "make_shape", "moe_route", "moe_permute", "moe_unpermute",
           "moe_grouped_gemm_fwd", "moe_grouped_gemm_bwd", "moe_layer_fwd", "moe_layer_bwd",
           "moe_workspace_bytes", "moe_status_str", "_native"]
