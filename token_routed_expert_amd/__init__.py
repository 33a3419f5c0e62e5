"""One GPU's routed-expert (mixture-of-experts) layer for AMD MI355X (gfx950).

The compute path is the HIP library libtre_moe.so (C ABI in include/moe.h);
this package only marshals torch tensors into its calls.
"""
from . import _native
from .ops import (E4M3Weights, MXWeights, MoeError, make_shape, moe_aux_loss, moe_combine_bwd,
                  moe_quantize_rows_mx, moe_quantize_weights_mx, moe_quantize_token_blocks_mx,
                  moe_permute_mx, moe_grouped_gemm_fwd_mx, moe_grouped_gemm_bwd_mx,
                  moe_row_probs, moe_grouped_gemm_fwd_rowscaled, moe_grouped_gemm_bwd_rowscaled,
                  moe_grouped_gemm_bwd, moe_route_bwd, moe_grouped_gemm_fwd_gather,
                  moe_grouped_gemm_bwd_gather, moe_route_aux, moe_aux_loss_final,
                  moe_grouped_gemm_bwd_e4m3, moe_grouped_gemm_fwd, moe_grouped_gemm_fwd_e4m3,
                  moe_layer_bwd, moe_layer_fwd, moe_permute, moe_permute_e4m3, moe_permute_noalloc,
                  moe_quantize_rows, moe_quantize_token_blocks, moe_quantize_weights, moe_route,
                  moe_status_str, moe_token_block_capacity, moe_unpermute, moe_workspace_bytes,
                  moe_probe_mfma, moe_quantize_token_blocks_with_rows,
                  moe_quantize_token_blocks_with_rows_mx)

__all__ = ["MoeError", "make_shape", "moe_route", "moe_permute", "moe_unpermute",
           "moe_grouped_gemm_fwd", "moe_grouped_gemm_bwd", "moe_layer_fwd", "moe_layer_bwd",
           "moe_workspace_bytes", "moe_status_str", "moe_quantize_rows", "moe_quantize_weights",
           "moe_token_block_capacity", "moe_quantize_token_blocks", "moe_permute_e4m3",
           "moe_grouped_gemm_fwd_e4m3", "moe_grouped_gemm_bwd_e4m3", "E4M3Weights", "moe_aux_loss",
           "moe_combine_bwd", "moe_route_bwd", "moe_row_probs", "moe_grouped_gemm_fwd_rowscaled",
           "moe_grouped_gemm_bwd_rowscaled", "MXWeights", "moe_quantize_rows_mx",
           "moe_quantize_weights_mx", "moe_quantize_token_blocks_mx", "moe_permute_mx",
           "moe_grouped_gemm_fwd_mx", "moe_grouped_gemm_bwd_mx", "moe_probe_mfma",
           "moe_permute_noalloc", "moe_grouped_gemm_fwd_gather",
           "moe_grouped_gemm_bwd_gather", "moe_route_aux",
           "moe_aux_loss_final", "moe_quantize_token_blocks_with_rows",
           "moe_quantize_token_blocks_with_rows_mx", "_native"]
