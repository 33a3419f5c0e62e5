"""ctypes view of libtre_moe.so: the structs and prototypes of include/moe.h.

Loading fails loudly when the library has not been built; there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes as C
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtre_moe.so")

MOE_OK, MOE_ERR_INVALID, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16, MOE_E4M3, MOE_MXFP8 = 0, 1, 2, 3
(MOE_WS_PERMUTE, MOE_WS_GEMM_FWD, MOE_WS_GEMM_BWD, MOE_WS_LAYER_FWD,
 MOE_WS_LAYER_BWD, MOE_WS_AUX_LOSS, MOE_WS_GEMM_BWD_ROWSCALED,
 MOE_WS_LAYER_BWD_ROWSCALED) = range(8)


class moe_shape(C.Structure):
    _fields_ = [("T", C.c_int64), ("d", C.c_int64), ("E", C.c_int64), ("k", C.c_int64),
                ("f", C.c_int64), ("f_shared", C.c_int64), ("dtype", C.c_int32),
                ("reserved", C.c_int32)]


_IO_FIELDS = [
    "logits", "x", "W1", "W3", "W2", "Ws1", "Ws3", "Ws2", "dY",
    "topk_idx", "topk_prob", "counts", "offsets", "row_of", "token_of",
    "xp", "ab", "h", "o", "s_ab", "s_h", "ys", "y",
    "dO", "dab", "dXp", "s_dab", "dXs", "dX", "dW1", "dW3", "dW2", "dWs1", "dWs3", "dWs2",
]


# e4m3 layers: `wq` points to a moe_e4m3_weights struct; the rest are tensors
_IO_FIELDS_E4M3 = ["wq", "xq", "xs", "xpq", "xps"]
# router gradient (optional)
_IO_FIELDS_ROUTER = ["aux_loss", "dprob", "dlogits"]


class moe_layer_io(C.Structure):
    _fields_ = ([(n, C.c_void_p) for n in _IO_FIELDS + _IO_FIELDS_E4M3 + _IO_FIELDS_ROUTER]
                + [("aux_alpha", C.c_float), ("row_prob", C.c_void_p),
                   ("memory_efficient", C.c_int32), ("wmx", C.c_void_p),
                   ("fused_permute", C.c_int32)])


IO_FIELDS = tuple(_IO_FIELDS + _IO_FIELDS_E4M3[1:] + _IO_FIELDS_ROUTER + ["row_prob"])


class moe_mx_weights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in
                ("W1", "W3", "W2", "W1t", "W3t", "W2t", "W1s", "W3s", "W2s", "W1ts", "W3ts", "W2ts")]


class moe_e4m3_weights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in
                ("W1", "W3", "W2", "W1t", "W3t", "W2t", "W1s", "W3s", "W2s")]

_P = C.c_void_p
_I64 = C.c_int64
_SH = C.POINTER(moe_shape)
_PROTOS = {
    "moe_route": (C.c_int, [_P, _I64, _I64, _I64, _P, _P, _P]),
    "moe_permute": (C.c_int, [_SH, _P, _P, _P, C.c_int, _P, _P, _P, _P, _P, _P, C.c_size_t, _P]),
    "moe_permute_noalloc": (C.c_int, [_SH, _P, _P, _P, C.c_int, _P, _P, _P, _P, _P, _P]),
    "moe_unpermute": (C.c_int, [_SH, _P, _P, _P, _P, _P, _P]),
    "moe_grouped_gemm_fwd": (C.c_int, [_SH, _P, _P, _P, _P, _P, _P, _P, _P, _P, C.c_size_t, _P]),
    "moe_grouped_gemm_bwd": (C.c_int, [_SH, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                       _P, C.c_size_t, _P]),
    "moe_grouped_gemm_fwd_gather": (C.c_int, [_SH, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                              C.c_size_t, _P]),
    "moe_grouped_gemm_bwd_gather": (C.c_int, [_SH] + [_P] * 15 + [C.c_size_t, _P]),
    "moe_layer_fwd": (C.c_int, [_SH, C.POINTER(moe_layer_io), _P, C.c_size_t, _P]),
    "moe_layer_bwd": (C.c_int, [_SH, C.POINTER(moe_layer_io), _P, C.c_size_t, _P]),
    "moe_quantize_rows": (C.c_int, [_P, C.c_int32, _I64, _I64, _P, _P, _P]),
    "moe_quantize_weights": (C.c_int, [_P, _I64, _I64, _I64, _P, _P, _P, _P]),
    "moe_token_block_capacity": (C.c_int64, [_I64, _I64]),
    "moe_quantize_token_blocks": (C.c_int, [_P, _I64, _I64, _P, _P, _I64, _P, _P, _P, _P]),
    "moe_quantize_token_blocks_with_rows": (C.c_int, [_P, _I64, _I64, _P, _P, _I64, _P, _P, _P, _P, _P,
                                                      _P]),
    "moe_permute_e4m3": (C.c_int, [_SH, _P, _P, _P, C.c_int, _P, _P, _P, _P, _P, _P, _P,
                                   C.c_size_t, _P]),
    "moe_grouped_gemm_fwd_e4m3": (C.c_int, [_SH, _P, _P, _P, C.POINTER(moe_e4m3_weights), _P, _P,
                                            _P, _P, C.c_size_t, _P]),
    "moe_grouped_gemm_bwd_e4m3": (C.c_int, [_SH, _P, _P, _P, _P, _P, _P,
                                            C.POINTER(moe_e4m3_weights), _P, _P, _P, _P, _P, _P,
                                            C.c_size_t, _P]),
    "moe_quantize_rows_mx": (C.c_int, [_P, C.c_int32, _I64, _I64, _P, _P, _P]),
    "moe_quantize_weights_mx": (C.c_int, [_P, _I64, _I64, _I64, _P, _P, _P, _P, _P]),
    "moe_quantize_token_blocks_mx": (C.c_int, [_P, _I64, _I64, _P, _P, _I64, _P, _P, _P, _P]),
    "moe_quantize_token_blocks_with_rows_mx": (C.c_int, [_P, _I64, _I64, _P, _P, _I64, _P, _P, _P, _P,
                                                         _P, _P]),
    "moe_permute_mx": (C.c_int, [_SH, _P, _P, _P, C.c_int, _P, _P, _P, _P, _P, _P, _P,
                                 C.c_size_t, _P]),
    "moe_grouped_gemm_fwd_mx": (C.c_int, [_SH, _P, _P, _P, C.POINTER(moe_mx_weights), _P, _P,
                                          _P, _P, C.c_size_t, _P]),
    "moe_grouped_gemm_bwd_mx": (C.c_int, [_SH, _P, _P, _P, _P, _P, _P,
                                          C.POINTER(moe_mx_weights), _P, _P, _P, _P, _P, _P,
                                          C.c_size_t, _P]),
    "moe_aux_loss": (C.c_int, [_P, _I64, _I64, _I64, _P, C.c_float, _P, _P, C.c_size_t, _P]),
    "moe_route_aux": (C.c_int, [_P, _I64, _I64, _I64, _P, _P, _P, C.c_size_t, _P]),
    "moe_aux_loss_final": (C.c_int, [_P, _I64, _I64, _I64, _P, C.c_float, _P, _P]),
    "moe_combine_bwd": (C.c_int, [_SH, _P, _P, _P, _P, _P, _P, _P]),
    "moe_route_bwd": (C.c_int, [_P, _I64, _I64, _I64, _P, _P, _P, _P, C.c_float, C.c_float, _P,
                                _P]),
    "moe_row_probs": (C.c_int, [_SH, _P, _P, _P, _P]),
    "moe_grouped_gemm_fwd_rowscaled": (C.c_int, [_SH] + [_P] * 10),
    "moe_grouped_gemm_bwd_rowscaled": (C.c_int, [_SH] + [_P] * 4 + [C.c_int32] + [_P] * 13
                                       + [C.c_size_t, _P]),
    "moe_workspace_bytes": (C.c_size_t, [_SH, C.c_int]),
    "moe_status_str": (C.c_char_p, [C.c_int]),
    "moe_probe_mfma": (C.c_int, [C.c_int, _I64, _P, _P, C.POINTER(C.c_int64), C.POINTER(C.c_int64),
                                 _P]),
}

_lib = None


def lib() -> C.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m token_routed_expert_amd.build` (no fallback exists)")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in _PROTOS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def exported_names():
    return tuple(_PROTOS)
