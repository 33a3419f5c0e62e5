"""fp64 oracle of the expert GEMMs with e4m3 block-quantised operands.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages run the expert GEMMs in FP8 with blockwise scaling and keep the
router in high precision ("Scalable Training of Mixture-of-Experts Models with
Megatron Core", gist.science German technical summary, section 2 E; French
summary, section 2 E).  Reading used (the quantiser itself is in
oracle/e4m3.py):

* every GEMM operand is quantised, then dequantised exactly (code * scale in
  fp64), and the product of the dequantised operands is taken in fp64;
* forward and data-gradient products quantise activations and gradients in
  1 x 128 blocks along the contraction (rows of xp, h, dO and [da|db]) and
  weights in 128 x 128 tiles of each expert's W1, W3 (d x f) and W2 (f x d),
  the same tiles serving the transposed products;
* weight-gradient products quantise both operands in 128-row token blocks per
  column, restarting at every expert's first row;
* the SwiGLU forward (h = silu(a) b) and backward epilogues use the unquantised
  a, b of the forward product, exactly as in oracle/moe.py.

Each product takes its input activations as values (fp32-representable, e.g.
bf16 tensors read back from the device), so a test can feed the same stored
intermediates to the oracle and to the device ("run on the same quantised
inputs"); layer_fwd_e4m3 / layer_bwd_e4m3 chain the products on the oracle's
own intermediates.
"""
from __future__ import annotations

import numpy as np

from .e4m3 import (dequant_rows, dequant_tiles, dequant_token_blocks, quant_rows, quant_tiles,
                   quant_token_blocks)
from .moe import combine, permute_map, permute_scaled, route, sigmoid, silu

__all__ = ["quant_expert_weights", "dequant_expert_weights", "fc1_fwd_e4m3", "fc2_fwd_e4m3",
           "fc2_dgrad_e4m3", "fc1_dgrad_e4m3", "wgrad_e4m3", "layer_fwd_e4m3",
           "layer_bwd_e4m3"]


def quant_expert_weights(W):
    """128 x 128 tiles of every expert matrix W [E][R][C]: codes [E][R][C],
    scales [E][R/128][C/128]."""
    W = np.asarray(W, dtype=np.float32)
    out = [quant_tiles(W[e]) for e in range(W.shape[0])]
    return np.stack([c for c, _ in out]), np.stack([s for _, s in out])


def dequant_expert_weights(codes, scales):
    return np.stack([dequant_tiles(codes[e], scales[e]) for e in range(codes.shape[0])])


def _segments(offsets):
    for e in range(len(offsets) - 1):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 > r0:
            yield e, slice(r0, r1)


def fc1_fwd_e4m3(xpq, xps, offsets, W1d, W3d):
    """a = xp W1, b = xp W3 per expert from the quantised rows (codes xpq,
    scales xps) and dequantised weights W1d, W3d [E][d][f]."""
    X = dequant_rows(xpq, xps)
    P, f = X.shape[0], W1d.shape[2]
    a = np.zeros((P, f)); b = np.zeros((P, f))
    for e, R in _segments(offsets):
        a[R] = X[R] @ W1d[e]
        b[R] = X[R] @ W3d[e]
    return a, b


def fc2_fwd_e4m3(h, offsets, W2d):
    """o = Q(h) W2 per expert; h [P][f] quantised 1 x 128 along f."""
    H = dequant_rows(*quant_rows(h))
    o = np.zeros((H.shape[0], W2d.shape[2]))
    for e, R in _segments(offsets):
        o[R] = H[R] @ W2d[e]
    return o


def fc2_dgrad_e4m3(dO, a, b, offsets, W2d):
    """dH = Q(dO) W2^T per expert, then the SwiGLU backward with s = sigmoid(a):
    da = dH b s (1 + a (1 - s)), db = dH silu(a)."""
    G = dequant_rows(*quant_rows(dO))
    a = np.asarray(a, np.float64); b = np.asarray(b, np.float64)
    dH = np.zeros_like(a)
    for e, R in _segments(offsets):
        dH[R] = G[R] @ W2d[e].T
    s = sigmoid(a)
    return dH * b * s * (1.0 + a * (1.0 - s)), dH * silu(a)


def fc1_dgrad_e4m3(dab, offsets, W1d, W3d):
    """dXp = Q([da|db]) [W1|W3]^T per expert; dab [P][2f] quantised 1 x 128 along 2f."""
    D = dequant_rows(*quant_rows(dab))
    f = W1d.shape[2]
    dXp = np.zeros((D.shape[0], W1d.shape[1]))
    for e, R in _segments(offsets):
        dXp[R] = D[R, :f] @ W1d[e].T + D[R, f:] @ W3d[e].T
    return dXp


def wgrad_e4m3(A, B, offsets):
    """dW_e = Q(A_e)^T Q(B_e) per expert, both quantised in 128-row token
    blocks per column; A [P][M], B [P][N] -> [E][M][N], zero for empty experts."""
    Ad = dequant_token_blocks(*quant_token_blocks(A, offsets), offsets)
    Bd = dequant_token_blocks(*quant_token_blocks(B, offsets), offsets)
    E = len(offsets) - 1
    dW = np.zeros((E, Ad.shape[1], Bd.shape[1]))
    for e, R in _segments(offsets):
        dW[e] = Ad[R].T @ Bd[R]
    return dW


def layer_fwd_e4m3(logits, x, W1, W3, W2, k):
    """Route, quantise x rows, permute codes and scales, e4m3 experts, combine,
    on the oracle's own intermediates.  W1, W3, W2 are the fp32 masters."""
    E = W1.shape[0]
    idx, p = route(logits, k)
    counts, offsets, row_of, token_of = permute_map(idx, E)
    xq, xs = quant_rows(x)
    xpq, xps = xq[token_of], xs[token_of]
    W1q, W1s = quant_expert_weights(W1); W3q, W3s = quant_expert_weights(W3)
    W2q, W2s = quant_expert_weights(W2)
    W1d, W3d, W2d = (dequant_expert_weights(c, s) for c, s in
                     ((W1q, W1s), (W3q, W3s), (W2q, W2s)))
    a, b = fc1_fwd_e4m3(xpq, xps, offsets, W1d, W3d)
    h = silu(a) * b
    o = fc2_fwd_e4m3(h, offsets, W2d)
    return dict(idx=idx, p=p, counts=counts, offsets=offsets, row_of=row_of, token_of=token_of,
                xq=xq, xs=xs, xpq=xpq, xps=xps, a=a, b=b, h=h, o=o, W1d=W1d, W3d=W3d, W2d=W2d,
                y=combine(o, row_of, p))


def layer_bwd_e4m3(st, x, dY):
    """Backward of layer_fwd_e4m3: dO = p dY permuted, e4m3 data and weight
    gradients, dX = un-permuted sum of dXp."""
    dO = permute_scaled(np.asarray(dY, np.float64), st["row_of"], st["p"])
    off = st["offsets"]
    da, db = fc2_dgrad_e4m3(dO, st["a"], st["b"], off, st["W2d"])
    dab = np.concatenate([da, db], axis=1)
    dXp = fc1_dgrad_e4m3(dab, off, st["W1d"], st["W3d"])
    dW2 = wgrad_e4m3(st["h"], dO, off)
    xp = np.asarray(x, np.float64)[st["token_of"]]
    dW13 = wgrad_e4m3(xp, dab, off)
    f = st["a"].shape[1]
    return dict(dO=dO, da=da, db=db, dXp=dXp, dW2=dW2, dW1=dW13[:, :, :f], dW3=dW13[:, :, f:],
                dX=combine(dXp, st["row_of"]))
