"""Python entry points with the names of the C ABI (include/moe.h).

Argument marshalling only: torch tensors supply device memory (data_ptr) and
the current HIP stream; every step runs in the library's kernels.  Each call
raises MoeError on a non-zero status.  Output tensors are passed in by the
caller, as in the C ABI.
"""
from __future__ import annotations

import ctypes as C

import torch

from . import _native as N


class MoeError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        name = N.lib().moe_status_str(status).decode()
        super().__init__(f"{call} returned {name} ({status})")


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"expected a torch.Tensor, got {type(t)}")
    if not t.is_contiguous():
        raise ValueError("tensors passed to the MoE library must be contiguous")
    return C.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def _check(status, call):
    if status != N.MOE_OK:
        raise MoeError(status, call)


def make_shape(T, d, E, k, f, f_shared=0, dtype="bf16") -> N.moe_shape:
    code = {"f32": N.MOE_F32, "bf16": N.MOE_BF16}[dtype]
    return N.moe_shape(int(T), int(d), int(E), int(k), int(f), int(f_shared), code, 0)


def moe_workspace_bytes(sh: N.moe_shape, kind: int) -> int:
    return int(N.lib().moe_workspace_bytes(C.byref(sh), kind))


def moe_status_str(status: int) -> str:
    return N.lib().moe_status_str(status).decode()


def moe_route(logits, k, topk_idx, topk_prob, stream=None):
    T, E = logits.shape
    _check(N.lib().moe_route(_ptr(logits), T, E, k, _ptr(topk_idx), _ptr(topk_prob),
                             _stream(stream)), "moe_route")


def moe_permute(sh, src, topk_idx, row_scale, build_map, counts, offsets, row_of, token_of, dst,
                ws, stream=None):
    ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(N.lib().moe_permute(C.byref(sh), _ptr(src), _ptr(topk_idx), _ptr(row_scale),
                               int(build_map), _ptr(counts), _ptr(offsets), _ptr(row_of),
                               _ptr(token_of), _ptr(dst), _ptr(ws), ws_bytes, _stream(stream)),
           "moe_permute")


def moe_unpermute(sh, src, row_of, topk_prob, add, dst, stream=None):
    _check(N.lib().moe_unpermute(C.byref(sh), _ptr(src), _ptr(row_of), _ptr(topk_prob), _ptr(add),
                                 _ptr(dst), _stream(stream)), "moe_unpermute")


def moe_grouped_gemm_fwd(sh, offsets, xp, W1, W3, W2, ab, h, o, stream=None):
    _check(N.lib().moe_grouped_gemm_fwd(C.byref(sh), _ptr(offsets), _ptr(xp), _ptr(W1), _ptr(W3),
                                        _ptr(W2), _ptr(ab), _ptr(h), _ptr(o), None, 0,
                                        _stream(stream)), "moe_grouped_gemm_fwd")


def moe_grouped_gemm_bwd(sh, offsets, xp, ab, h, dO, W1, W3, W2, dab, dXp, dW1, dW3, dW2,
                         stream=None):
    _check(N.lib().moe_grouped_gemm_bwd(C.byref(sh), _ptr(offsets), _ptr(xp), _ptr(ab), _ptr(h),
                                        _ptr(dO), _ptr(W1), _ptr(W3), _ptr(W2), _ptr(dab),
                                        _ptr(dXp), _ptr(dW1), _ptr(dW3), _ptr(dW2), None, 0,
                                        _stream(stream)), "moe_grouped_gemm_bwd")


def _io(buffers: dict) -> N.moe_layer_io:
    io = N.moe_layer_io()
    for name in N.IO_FIELDS:
        t = buffers.get(name)
        setattr(io, name, None if t is None else _ptr(t).value)
    return io


def moe_layer_fwd(sh, buffers: dict, ws, stream=None):
    io = _io(buffers)
    _check(N.lib().moe_layer_fwd(C.byref(sh), C.byref(io), _ptr(ws), ws.numel() * ws.element_size(),
                                 _stream(stream)), "moe_layer_fwd")


def moe_layer_bwd(sh, buffers: dict, ws, stream=None):
    io = _io(buffers)
    _check(N.lib().moe_layer_bwd(C.byref(sh), C.byref(io), _ptr(ws), ws.numel() * ws.element_size(),
                                 _stream(stream)), "moe_layer_bwd")
