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

F32 = torch.float32
I32 = torch.int32


class MoeError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        name = N.lib().moe_status_str(status).decode()
        super().__init__(f"{call} returned {name} ({status})")


def _ptr(t, dtype=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"expected a torch.Tensor, got {type(t)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"expected a {dtype} tensor, got {t.dtype}")
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
    code = {"f32": N.MOE_F32, "bf16": N.MOE_BF16, "e4m3": N.MOE_E4M3, "mxfp8": N.MOE_MXFP8}[dtype]
    return N.moe_shape(int(T), int(d), int(E), int(k), int(f), int(f_shared), code, 0)


def moe_workspace_bytes(sh: N.moe_shape, kind: int) -> int:
    return int(N.lib().moe_workspace_bytes(C.byref(sh), kind))


def moe_status_str(status: int) -> str:
    return N.lib().moe_status_str(status).decode()


def moe_route(logits, k, topk_idx, topk_prob, stream=None):
    T, E = logits.shape
    _check(N.lib().moe_route(_ptr(logits, F32), T, E, k, _ptr(topk_idx, I32), _ptr(topk_prob, F32),
                             _stream(stream)), "moe_route")


def moe_permute(sh, src, topk_idx, row_scale, build_map, counts, offsets, row_of, token_of, dst,
                ws, stream=None):
    ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(N.lib().moe_permute(C.byref(sh), _ptr(src), _ptr(topk_idx, I32), _ptr(row_scale, F32),
                               int(build_map), _ptr(counts, I32), _ptr(offsets, I32),
                               _ptr(row_of, I32), _ptr(token_of, I32), _ptr(dst), _ptr(ws),
                               ws_bytes, _stream(stream)),
           "moe_permute")


def moe_permute_noalloc(sh, src, topk_idx, row_scale, build_map, counts, offsets, row_of,
                        token_of, dst, stream=None):
    _check(N.lib().moe_permute_noalloc(C.byref(sh), _ptr(src), _ptr(topk_idx, I32),
                                       _ptr(row_scale, F32), int(build_map), _ptr(counts, I32),
                                       _ptr(offsets, I32), _ptr(row_of, I32), _ptr(token_of, I32),
                                       _ptr(dst), _stream(stream)),
           "moe_permute_noalloc")


def moe_unpermute(sh, src, row_of, topk_prob, add, dst, stream=None):
    _check(N.lib().moe_unpermute(C.byref(sh), _ptr(src), _ptr(row_of, I32), _ptr(topk_prob, F32),
                                 _ptr(add), _ptr(dst), _stream(stream)), "moe_unpermute")


def moe_grouped_gemm_fwd(sh, offsets, xp, W1, W3, W2, ab, h, o, stream=None):
    _check(N.lib().moe_grouped_gemm_fwd(C.byref(sh), _ptr(offsets, I32), _ptr(xp), _ptr(W1),
                                        _ptr(W3), _ptr(W2), _ptr(ab), _ptr(h), _ptr(o), None, 0,
                                        _stream(stream)), "moe_grouped_gemm_fwd")


def moe_grouped_gemm_bwd(sh, offsets, xp, ab, h, dO, W1, W3, W2, dab, dXp, dW1, dW3, dW2,
                         stream=None):
    _check(N.lib().moe_grouped_gemm_bwd(C.byref(sh), _ptr(offsets, I32), _ptr(xp), _ptr(ab),
                                        _ptr(h), _ptr(dO), _ptr(W1), _ptr(W3), _ptr(W2),
                                        _ptr(dab), _ptr(dXp), _ptr(dW1), _ptr(dW3), _ptr(dW2),
                                        None, 0, _stream(stream)), "moe_grouped_gemm_bwd")


def moe_grouped_gemm_fwd_gather(sh, offsets, token_of, x, W1, W3, W2, ab, h, o, stream=None):
    """moe_grouped_gemm_fwd with fc1 reading row token_of[r] of x (no xp)."""
    _check(N.lib().moe_grouped_gemm_fwd_gather(C.byref(sh), _ptr(offsets, I32), _ptr(token_of, I32),
                                               _ptr(x), _ptr(W1), _ptr(W3), _ptr(W2), _ptr(ab),
                                               _ptr(h), _ptr(o), None, 0, _stream(stream)),
           "moe_grouped_gemm_fwd_gather")


def moe_grouped_gemm_bwd_gather(sh, offsets, token_of, x, ab, h, dO, W1, W3, W2, dab, dXp, dW1,
                                dW3, dW2, stream=None):
    """moe_grouped_gemm_bwd with the fc1 weight gradient reading row
    token_of[r] of x (no xp)."""
    _check(N.lib().moe_grouped_gemm_bwd_gather(C.byref(sh), _ptr(offsets, I32), _ptr(token_of, I32),
                                               _ptr(x), _ptr(ab), _ptr(h), _ptr(dO), _ptr(W1),
                                               _ptr(W3), _ptr(W2), _ptr(dab), _ptr(dXp), _ptr(dW1),
                                               _ptr(dW3), _ptr(dW2), None, 0, _stream(stream)),
           "moe_grouped_gemm_bwd_gather")


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def moe_quantize_rows(src, codes, scales, stream=None):
    """1 x 128 e4m3 blocks along the rows of a bf16 or fp32 matrix."""
    rows, cols = src.shape
    code = {torch.bfloat16: N.MOE_BF16, torch.float32: N.MOE_F32}[src.dtype]
    _check(N.lib().moe_quantize_rows(_ptr(src), code, rows, cols, _ptr(codes), _ptr(scales),
                                     _stream(stream)), "moe_quantize_rows")


def moe_quantize_weights(W, codes, codes_t, scales, stream=None):
    """128 x 128 e4m3 tiles of fp32 matrices W [E][R][C]."""
    E, R, Cc = W.shape
    _check(N.lib().moe_quantize_weights(_ptr(W), E, R, Cc, _ptr(codes), _ptr(codes_t), _ptr(scales),
                                        _stream(stream)), "moe_quantize_weights")


def moe_token_block_capacity(P, E) -> int:
    return int(N.lib().moe_token_block_capacity(int(P), int(E)))


def moe_quantize_token_blocks(offsets, E, P, src, src_row, blk, codes, scales, stream=None):
    """Per-expert 128-row e4m3 blocks of a bf16 [.][C] matrix: codes [P][C], scales [cap][C]."""
    Cc = src.shape[1]
    _check(N.lib().moe_quantize_token_blocks(_ptr(offsets, I32), int(E), int(P), _ptr(src),
                                             _ptr(src_row, I32), Cc, _ptr(blk, I32),
                                             _ptr(codes), _ptr(scales, F32), _stream(stream)),
           "moe_quantize_token_blocks")


def moe_quantize_token_blocks_with_rows(offsets, E, P, src, src_row, blk, codes, scales, row_codes,
                                        row_scales, stream=None):
    """moe_quantize_token_blocks plus the 1 x 128 row blocks of the same rows, in one pass."""
    Cc = src.shape[1]
    _check(N.lib().moe_quantize_token_blocks_with_rows(
        _ptr(offsets, I32), int(E), int(P), _ptr(src), _ptr(src_row, I32), Cc, _ptr(blk, I32),
        _ptr(codes), _ptr(scales, F32), _ptr(row_codes), _ptr(row_scales, F32), _stream(stream)),
        "moe_quantize_token_blocks_with_rows")


def moe_permute_e4m3(sh, codes, scales, topk_idx, build_map, counts, offsets, row_of, token_of,
                     dst_codes, dst_scales, ws, stream=None):
    _check(N.lib().moe_permute_e4m3(C.byref(sh), _ptr(codes), _ptr(scales, F32),
                                    _ptr(topk_idx, I32), int(build_map), _ptr(counts, I32),
                                    _ptr(offsets, I32), _ptr(row_of, I32), _ptr(token_of, I32),
                                    _ptr(dst_codes), _ptr(dst_scales, F32), _ptr(ws),
                                    _nbytes(ws), _stream(stream)), "moe_permute_e4m3")


class E4M3Weights:
    """The moe_e4m3_weights struct over torch tensors (kept alive here)."""

    NAMES = ("W1", "W3", "W2", "W1t", "W3t", "W2t", "W1s", "W3s", "W2s")

    def __init__(self, tensors: dict):
        # the transposed codes (W1t, W3t, W2t) are optional: the library does not read them
        self.tensors = {n: tensors.get(n) for n in self.NAMES}
        self.struct = N.moe_e4m3_weights(*[(_ptr(self.tensors[n]) or C.c_void_p(0)).value
                                           for n in self.NAMES])

    def __getitem__(self, name):
        return self.tensors[name]


def moe_grouped_gemm_fwd_e4m3(sh, offsets, xpq, xps, wq: E4M3Weights, ab, h, o, ws, stream=None):
    _check(N.lib().moe_grouped_gemm_fwd_e4m3(C.byref(sh), _ptr(offsets, I32), _ptr(xpq),
                                             _ptr(xps, F32), C.byref(wq.struct), _ptr(ab), _ptr(h),
                                             _ptr(o), _ptr(ws), _nbytes(ws), _stream(stream)),
           "moe_grouped_gemm_fwd_e4m3")


def moe_grouped_gemm_bwd_e4m3(sh, offsets, token_of, x, ab, h, dO, wq: E4M3Weights, dab, dXp, dW1,
                              dW3, dW2, ws, stream=None):
    _check(N.lib().moe_grouped_gemm_bwd_e4m3(C.byref(sh), _ptr(offsets, I32),
                                             _ptr(token_of, I32), _ptr(x), _ptr(ab), _ptr(h),
                                             _ptr(dO), C.byref(wq.struct),
                                             _ptr(dab), _ptr(dXp), _ptr(dW1), _ptr(dW3), _ptr(dW2),
                                             _ptr(ws), _nbytes(ws), _stream(stream)),
           "moe_grouped_gemm_bwd_e4m3")


U8 = torch.uint8


def moe_quantize_rows_mx(src, codes, scales, stream=None):
    """1 x 32 MXFP8 blocks along the rows of a bf16 or fp32 matrix (E8M0 scale bytes)."""
    rows, cols = src.shape
    code = {torch.bfloat16: N.MOE_BF16, torch.float32: N.MOE_F32}[src.dtype]
    _check(N.lib().moe_quantize_rows_mx(_ptr(src), code, rows, cols, _ptr(codes, U8),
                                        _ptr(scales, U8), _stream(stream)), "moe_quantize_rows_mx")


def moe_quantize_weights_mx(W, codes, scales, codes_t, scales_t, stream=None):
    """Both MXFP8 orientations of fp32 matrices W [E][R][C]."""
    E, R, Cc = W.shape
    _check(N.lib().moe_quantize_weights_mx(_ptr(W, F32), E, R, Cc, _ptr(codes, U8),
                                           _ptr(scales, U8), _ptr(codes_t, U8),
                                           _ptr(scales_t, U8), _stream(stream)),
           "moe_quantize_weights_mx")


def moe_quantize_token_blocks_mx(offsets, E, P, src, src_row, blk, codes, scales, stream=None):
    """Per-expert token blocks with 32-row MXFP8 scale blocks: codes [P][C], bytes [cap][C][4]."""
    Cc = src.shape[1]
    _check(N.lib().moe_quantize_token_blocks_mx(_ptr(offsets, I32), int(E), int(P), _ptr(src),
                                                _ptr(src_row, I32), Cc, _ptr(blk, I32),
                                                _ptr(codes, U8), _ptr(scales, U8),
                                                _stream(stream)), "moe_quantize_token_blocks_mx")


def moe_quantize_token_blocks_with_rows_mx(offsets, E, P, src, src_row, blk, codes, scales,
                                           row_codes, row_scales, stream=None):
    """moe_quantize_token_blocks_mx plus the 1 x 32 row blocks of the same rows, in one pass."""
    Cc = src.shape[1]
    _check(N.lib().moe_quantize_token_blocks_with_rows_mx(
        _ptr(offsets, I32), int(E), int(P), _ptr(src), _ptr(src_row, I32), Cc, _ptr(blk, I32),
        _ptr(codes, U8), _ptr(scales, U8), _ptr(row_codes, U8), _ptr(row_scales, U8),
        _stream(stream)), "moe_quantize_token_blocks_with_rows_mx")


def moe_permute_mx(sh, codes, scales, topk_idx, build_map, counts, offsets, row_of, token_of,
                   dst_codes, dst_scales, ws, stream=None):
    _check(N.lib().moe_permute_mx(C.byref(sh), _ptr(codes, U8), _ptr(scales, U8),
                                  _ptr(topk_idx, I32), int(build_map), _ptr(counts, I32),
                                  _ptr(offsets, I32), _ptr(row_of, I32), _ptr(token_of, I32),
                                  _ptr(dst_codes, U8), _ptr(dst_scales, U8), _ptr(ws),
                                  _nbytes(ws), _stream(stream)), "moe_permute_mx")


class MXWeights:
    """The moe_mx_weights struct over torch tensors (kept alive here)."""

    NAMES = ("W1", "W3", "W2", "W1t", "W3t", "W2t", "W1s", "W3s", "W2s", "W1ts", "W3ts", "W2ts")

    def __init__(self, tensors: dict):
        self.tensors = {n: tensors[n] for n in self.NAMES}
        self.struct = N.moe_mx_weights(*[_ptr(self.tensors[n], U8).value for n in self.NAMES])

    def __getitem__(self, name):
        return self.tensors[name]


def moe_grouped_gemm_fwd_mx(sh, offsets, xpq, xps, w: MXWeights, ab, h, o, ws, stream=None):
    _check(N.lib().moe_grouped_gemm_fwd_mx(C.byref(sh), _ptr(offsets, I32), _ptr(xpq, U8),
                                           _ptr(xps, U8), C.byref(w.struct), _ptr(ab), _ptr(h),
                                           _ptr(o), _ptr(ws), _nbytes(ws), _stream(stream)),
           "moe_grouped_gemm_fwd_mx")


def moe_grouped_gemm_bwd_mx(sh, offsets, token_of, x, ab, h, dO, w: MXWeights, dab, dXp, dW1, dW3,
                            dW2, ws, stream=None):
    _check(N.lib().moe_grouped_gemm_bwd_mx(C.byref(sh), _ptr(offsets, I32), _ptr(token_of, I32),
                                           _ptr(x), _ptr(ab), _ptr(h), _ptr(dO), C.byref(w.struct),
                                           _ptr(dab), _ptr(dXp), _ptr(dW1), _ptr(dW3), _ptr(dW2),
                                           _ptr(ws), _nbytes(ws), _stream(stream)),
           "moe_grouped_gemm_bwd_mx")


def _io(buffers: dict) -> N.moe_layer_io:
    io = N.moe_layer_io()
    for name in N.IO_FIELDS:
        t = buffers.get(name)
        setattr(io, name, None if t is None else _ptr(t).value)
    wq = buffers.get("wq")
    if wq is not None:
        io.wq = C.cast(C.pointer(wq.struct), C.c_void_p).value
    wmx = buffers.get("wmx")
    if wmx is not None:
        io.wmx = C.cast(C.pointer(wmx.struct), C.c_void_p).value
    io.aux_alpha = float(buffers.get("aux_alpha", 0.0))
    io.memory_efficient = int(buffers.get("memory_efficient", 0))
    io.fused_permute = int(buffers.get("fused_permute", 0))
    return io


def moe_row_probs(sh, row_of, topk_prob, row_prob, stream=None):
    """row_prob[row_of[t][j]] = topk_prob[t][j]."""
    _check(N.lib().moe_row_probs(C.byref(sh), _ptr(row_of, I32), _ptr(topk_prob, F32),
                                 _ptr(row_prob, F32), _stream(stream)), "moe_row_probs")


def moe_grouped_gemm_fwd_rowscaled(sh, offsets, xp, W1, W3, W2, row_prob, ab, h, o, stream=None):
    """Expert forward with h = p * silu(a) * b (probabilities applied before W2)."""
    _check(N.lib().moe_grouped_gemm_fwd_rowscaled(
        C.byref(sh), _ptr(offsets, I32), _ptr(xp), _ptr(W1), _ptr(W3), _ptr(W2),
        _ptr(row_prob, F32), _ptr(ab), _ptr(h), _ptr(o), _stream(stream)),
        "moe_grouped_gemm_fwd_rowscaled")


def moe_grouped_gemm_bwd_rowscaled(sh, offsets, xp, ab, h, dO, W1, W3, W2, row_prob, dab, dXp,
                                   dW1, dW3, dW2, row_of, dprob, ws, recompute_h=False,
                                   stream=None):
    """Backward of the row-scaled forward for the unscaled permuted dO; dprob is
    [P] in row order (row_of None) or [T][k]; recompute_h refills h first."""
    _check(N.lib().moe_grouped_gemm_bwd_rowscaled(
        C.byref(sh), _ptr(offsets, I32), _ptr(xp), _ptr(ab), _ptr(h), int(bool(recompute_h)),
        _ptr(dO), _ptr(W1),
        _ptr(W3), _ptr(W2), _ptr(row_prob, F32), _ptr(dab), _ptr(dXp), _ptr(dW1), _ptr(dW3),
        _ptr(dW2), _ptr(row_of, I32), _ptr(dprob, F32), _ptr(ws), _nbytes(ws), _stream(stream)),
        "moe_grouped_gemm_bwd_rowscaled")


def moe_aux_loss(logits, k, counts, alpha, loss, ws, stream=None):
    """Load-balancing loss (device scalar `loss`) from logits [T][E] and counts [E]."""
    T, E = logits.shape
    _check(N.lib().moe_aux_loss(_ptr(logits, F32), T, E, int(k), _ptr(counts, I32), float(alpha),
                                _ptr(loss, F32), _ptr(ws), _nbytes(ws), _stream(stream)),
           "moe_aux_loss")


def moe_route_aux(logits, k, topk_idx, topk_prob, ws, stream=None):
    """moe_route plus the load-balancing loss's column sums (into ws)."""
    T, E = logits.shape
    _check(N.lib().moe_route_aux(_ptr(logits, F32), T, E, k, _ptr(topk_idx, I32),
                                 _ptr(topk_prob, F32), _ptr(ws), _nbytes(ws), _stream(stream)),
           "moe_route_aux")


def moe_aux_loss_final(ws, T, E, k, counts, alpha, loss, stream=None):
    """The load-balancing loss from moe_route_aux's column sums and the counts."""
    _check(N.lib().moe_aux_loss_final(_ptr(ws), int(T), int(E), int(k), _ptr(counts, I32),
                                      float(alpha), _ptr(loss, F32), _stream(stream)),
           "moe_aux_loss_final")


def moe_combine_bwd(sh, dY, o, row_of, topk_prob, dO, dprob, stream=None):
    """dO = p * dY permuted, and dprob[t][j] = <dY[t], o[row_of[t][j]]>."""
    _check(N.lib().moe_combine_bwd(C.byref(sh), _ptr(dY), _ptr(o), _ptr(row_of, I32),
                                   _ptr(topk_prob, F32), _ptr(dO), _ptr(dprob, F32),
                                   _stream(stream)), "moe_combine_bwd")


def moe_route_bwd(logits, k, topk_idx, topk_prob, dprob, counts, alpha, aux_scale, dlogits,
                  stream=None):
    """Router gradient dlogits [T][E]: top-k softmax Jacobian + aux_scale * load-balancing term."""
    T, E = logits.shape
    _check(N.lib().moe_route_bwd(_ptr(logits, F32), T, E, int(k), _ptr(topk_idx, I32),
                                 _ptr(topk_prob, F32), _ptr(dprob, F32), _ptr(counts, I32),
                                 float(alpha), float(aux_scale), _ptr(dlogits, F32),
                                 _stream(stream)), "moe_route_bwd")


def moe_layer_fwd(sh, buffers: dict, ws, stream=None):
    io = _io(buffers)
    _check(N.lib().moe_layer_fwd(C.byref(sh), C.byref(io), _ptr(ws), ws.numel() * ws.element_size(),
                                 _stream(stream)), "moe_layer_fwd")


def moe_layer_bwd(sh, buffers: dict, ws, stream=None):
    io = _io(buffers)
    _check(N.lib().moe_layer_bwd(C.byref(sh), C.byref(io), _ptr(ws), ws.numel() * ws.element_size(),
                                 _stream(stream)), "moe_layer_bwd")


def moe_probe_mfma(dtype, iters, ticks, sink, stream=None):
    """Launches the matrix-core probe (dtype "bf16" or "e4m3") on the stream;
    `ticks` is a device uint64 tensor of 2 (int64 storage), `sink` a device
    float tensor of 1.  Returns (flop count of the launch, wall-clock kHz)."""
    code = {"bf16": N.MOE_BF16, "e4m3": N.MOE_E4M3}[dtype]
    flops, khz = C.c_int64(0), C.c_int64(0)
    _check(N.lib().moe_probe_mfma(code, int(iters), _ptr(ticks), _ptr(sink), C.byref(flops),
                                  C.byref(khz), _stream(stream)), "moe_probe_mfma")
    return int(flops.value), int(khz.value)
