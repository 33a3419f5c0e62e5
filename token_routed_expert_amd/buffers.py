"""Device buffers of one layer, allocated with torch (memory plumbing only)."""
from __future__ import annotations

import torch

from . import _native as N
from .ops import (E4M3Weights, MXWeights, make_shape, moe_quantize_weights,
                  moe_quantize_weights_mx, moe_workspace_bytes)


def layer_buffers(T, d, E, k, f, f_shared=0, dtype="bf16", device="cuda", inputs=None,
                  router_grad=False, aux_alpha=0.01, memory_efficient=False,
                  fused_permute=False):
    """Every buffer moe_layer_fwd/bwd touch, as a dict keyed like moe_layer_io.

    `inputs` (logits, x, W1, W3, W2, Ws1, Ws3, Ws2, dY) are used as given.
    router_grad: also the load-balancing loss (coefficient aux_alpha) and the
    router gradient (aux_loss, dprob, dlogits).
    memory_efficient: probabilities applied before W2 (row_prob [P]);
    2 also recomputes h in the backward.
    fused_permute: the experts read x through token_of; no xp buffer.
    Returns (shape, buffers, ws_fwd, ws_bwd).
    """
    sh = make_shape(T, d, E, k, f, f_shared, dtype)
    dt = torch.float32 if dtype == "f32" else torch.bfloat16  # e4m3 layers: bf16 activations
    P = T * k
    b = dict(inputs or {})

    def z(*shape, dtype=dt):
        return torch.empty(shape, dtype=dtype, device=device)

    b.update(topk_idx=z(T, k, dtype=torch.int32), topk_prob=z(T, k, dtype=torch.float32),
             counts=z(E, dtype=torch.int32), offsets=z(E + 1, dtype=torch.int32),
             row_of=z(T, k, dtype=torch.int32), token_of=z(P, dtype=torch.int32),
             xp=z(P, d), ab=z(P, 2 * f), h=z(P, f), o=z(P, d), y=z(T, d),
             dO=z(P, d), dab=z(P, 2 * f), dXp=z(P, d), dX=z(T, d),
             dW1=z(E, d, f), dW3=z(E, d, f), dW2=z(E, f, d))
    if dtype == "e4m3":
        u8 = torch.uint8
        b.pop("xp")
        b.update(xq=z(T, d, dtype=u8), xs=z(T, d // 128, dtype=torch.float32),
                 xpq=z(P, d, dtype=u8), xps=z(P, d // 128, dtype=torch.float32))
        if "W1" in b and b["W1"].dtype == torch.float32:
            b["wq"] = quantized_weights(b["W1"], b["W3"], b["W2"])
    if dtype == "mxfp8":
        u8 = torch.uint8
        b.pop("xp")
        b.update(xq=z(T, d, dtype=u8), xs=z(T, d // 32, dtype=u8),
                 xpq=z(P, d, dtype=u8), xps=z(P, d // 32, dtype=u8))
        if "W1" in b and b["W1"].dtype == torch.float32:
            b["wmx"] = quantized_weights_mx(b["W1"], b["W3"], b["W2"])
    if fused_permute:
        b.pop("xp", None)
        b["fused_permute"] = 1
    if f_shared:
        b.update(s_ab=z(T, 2 * f_shared), s_h=z(T, f_shared), ys=z(T, d), s_dab=z(T, 2 * f_shared),
                 dXs=z(T, d), dWs1=z(d, f_shared), dWs3=z(d, f_shared), dWs2=z(f_shared, d))
    ws_f_bytes = moe_workspace_bytes(sh, N.MOE_WS_LAYER_FWD)
    if router_grad:
        b.update(aux_loss=z(1, dtype=torch.float32), dprob=z(T, k, dtype=torch.float32),
                 dlogits=z(T, E, dtype=torch.float32), aux_alpha=float(aux_alpha))
        ws_f_bytes += moe_workspace_bytes(sh, N.MOE_WS_AUX_LOSS)
    ws_f = torch.empty(max(256, ws_f_bytes), dtype=torch.uint8, device=device)
    bwd_kind = N.MOE_WS_LAYER_BWD
    if memory_efficient:
        b.update(row_prob=z(P, dtype=torch.float32), memory_efficient=int(memory_efficient))
        bwd_kind = N.MOE_WS_LAYER_BWD_ROWSCALED
    ws_b = torch.empty(max(256, moe_workspace_bytes(sh, bwd_kind)), dtype=torch.uint8,
                       device=device)
    return sh, b, ws_f, ws_b


def quantized_weights(W1, W3, W2, stream=None, transposed=False) -> E4M3Weights:
    """e4m3 codes and 128 x 128 scales of fp32 expert weights (W1, W3
    [E][d][f], W2 [E][f][d]), made by moe_quantize_weights; transposed=True
    also writes the transposed codes (which the products do not read)."""
    E, d, f = W1.shape
    dev = W1.device
    t = {}
    for name, W, R, Cc in (("W1", W1, d, f), ("W3", W3, d, f), ("W2", W2, f, d)):
        t[name] = torch.empty(E, R, Cc, dtype=torch.uint8, device=dev)
        if transposed:
            t[name + "t"] = torch.empty(E, Cc, R, dtype=torch.uint8, device=dev)
        t[name + "s"] = torch.empty(E, R // 128, Cc // 128, dtype=torch.float32, device=dev)
    wq = E4M3Weights(t)
    requantize_weights(wq, W1, W3, W2, stream)
    return wq


def requantize_weights(wq, W1, W3, W2, stream=None):
    """Refresh wq (E4M3Weights or MXWeights) from the fp32 masters (e.g. after an
    optimizer step)."""
    for name, W in (("W1", W1), ("W3", W3), ("W2", W2)):
        if isinstance(wq, MXWeights):
            moe_quantize_weights_mx(W, wq[name], wq[name + "s"], wq[name + "t"], wq[name + "ts"],
                                    stream)
        else:
            moe_quantize_weights(W, wq[name], wq[name + "t"], wq[name + "s"], stream)  # t may be None


def quantized_weights_mx(W1, W3, W2, stream=None) -> MXWeights:
    """MXFP8 codes and E8M0 scale bytes of fp32 expert weights in both
    orientations, made by moe_quantize_weights_mx."""
    E, d, f = W1.shape
    dev = W1.device
    t = {}
    for name, W, R, Cc in (("W1", W1, d, f), ("W3", W3, d, f), ("W2", W2, f, d)):
        t[name] = torch.empty(E, R, Cc, dtype=torch.uint8, device=dev)
        t[name + "s"] = torch.empty(E, R, Cc // 32, dtype=torch.uint8, device=dev)
        t[name + "t"] = torch.empty(E, Cc, R, dtype=torch.uint8, device=dev)
        t[name + "ts"] = torch.empty(E, Cc, R // 32, dtype=torch.uint8, device=dev)
    wq = MXWeights(t)
    requantize_weights(wq, W1, W3, W2, stream)
    return wq
