"""MXFP8 oracle: e4m3 elements with one power-of-two (E8M0) scale per 32 values.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages name MXFP8 as the FP8 recipe of the Blackwell runs, beside the
blockwise recipe on Hopper ("Scalable Training of Mixture-of-Experts Models
with Megatron Core", gist.science French technical summary, section 2 E;
Spanish summary, section 2.4), without a definition.  The storage follows
the OCP Microscaling format: blocks of 32 consecutive values along the
contraction axis share an 8-bit exponent-only scale 2^s (E8M0 byte s + 127),
elements are OCP E4M3FN.  Reading used for the scale and the codes of a block
of fp32 values:

* amax = max |v|; s is the smallest integer with amax <= 448 * 2^s (the
  scale rounded up to a power of two, so no element saturates), clamped to
  [-127, 127]; an all-zero block has s = 0 and every code +0.  This departs
  from the OCP MX v1.0 reference conversion, which takes s = floor(log2 amax)
  - 8 and clamps elements above 448: with that rule a block whose largest
  magnitude lies in (448, 512) * 2^s loses up to 12.5 % on it, where the
  rounded-up scale keeps every element within half an e4m3 step, at the
  cost of one binade of resolution for blocks with amax in (1.75, 2) * 2^E;
* code(v) = E4M3(v * 2^-s), round to nearest, ties to even (the product is
  exact in fp32 except where it falls below 2^-126, where every code is 0);
  the sign is kept, so -0 and tiny negatives give 0x80;
* value = e4m3(code) * 2^s, exact in fp64.

Block layouts: rows of activations and gradients (xp, h, dO, [da db]) in 1 x
32 blocks along the row; each expert weight matrix twice, once in 1 x 32
blocks along its rows (the operand of the data-gradient products) and once
in 32 x 1 blocks along its columns, stored transposed (the operand of the
forward products); weight-gradient operands in 32-row blocks per column,
restarting at every expert's first row (codes keep the operand's [P][C]
shape; one scale per block and column).

Every GEMM of dequantised operands is a plain fp64 product (the hardware's
block-scaled MFMA multiplies exact block sums by 2^(s_A + s_B)).
"""
from __future__ import annotations

import numpy as np

from .e4m3 import e4m3_decode, e4m3_encode, token_block_offsets
from .moe import combine, permute_map, permute_scaled, route, sigmoid, silu

__all__ = ["MX_BLOCK", "mx_scale_exp", "quant_mx_rows", "dequant_mx_rows", "quant_mx_weights",
           "dequant_mx_weights", "quant_mx_token_blocks", "dequant_mx_token_blocks",
           "fc1_fwd_mx", "fc2_fwd_mx", "fc2_dgrad_mx", "fc1_dgrad_mx", "wgrad_mx",
           "layer_fwd_mx", "layer_bwd_mx"]

MX_BLOCK = 32


def mx_scale_exp(amax):
    """Smallest s with amax <= 448 * 2^s, clamped to [-127, 127]; 0 for amax == 0.

    amax = f * 2^E with f in [1, 2): 448 = 1.75 * 2^8, so s = E - 8 when
    f <= 1.75 and E - 7 otherwise.
    """
    a = np.asarray(amax, dtype=np.float64)
    m, e = np.frexp(a)                     # a = m 2^e, m in [0.5, 1)
    f, E = 2.0 * m, e - 1
    s = E - 8 + (f > 1.75)
    s = np.clip(s, -127, 127)
    return np.where(a == 0, 0, s).astype(np.int64)


def _mx_groups(V):
    """Quantise every vector along the last axis of V (length 32) as one
    block: codes uint8 (shape of V), E8M0 scale bytes (V.shape[:-1])."""
    V = np.asarray(V, dtype=np.float32)
    amax = np.max(np.abs(V), axis=-1)
    s = mx_scale_exp(amax)
    scaled = (V.astype(np.float64) * np.ldexp(1.0, -s)[..., None]).astype(np.float32)
    codes = e4m3_encode(scaled)
    codes[amax == 0] = 0
    return codes, (s + 127).astype(np.uint8)


def _scale_values(sbytes):
    return np.ldexp(1.0, np.asarray(sbytes, np.int64) - 127)


def quant_mx_rows(A):
    """1 x 32 blocks along the last axis: codes [R][K], scale bytes [R][K/32]."""
    A = np.asarray(A, dtype=np.float32)
    R, K = A.shape
    assert K % MX_BLOCK == 0
    codes, sb = _mx_groups(A.reshape(R, K // MX_BLOCK, MX_BLOCK))
    return codes.reshape(R, K), sb


def dequant_mx_rows(codes, sbytes):
    return e4m3_decode(codes) * np.repeat(_scale_values(sbytes), MX_BLOCK, axis=1)


def quant_mx_weights(W):
    """Both orientations of every expert matrix W [E][R][C]:
    codes [E][R][C] with scale bytes [E][R][C/32] (blocks along each row), and
    codes_t [E][C][R] with scale bytes [E][C][R/32] (blocks along each column,
    stored transposed)."""
    W = np.asarray(W, dtype=np.float32)
    rows = [quant_mx_rows(W[e]) for e in range(W.shape[0])]
    cols = [quant_mx_rows(np.ascontiguousarray(W[e].T)) for e in range(W.shape[0])]
    return (np.stack([c for c, _ in rows]), np.stack([s for _, s in rows]),
            np.stack([c for c, _ in cols]), np.stack([s for _, s in cols]))


def dequant_mx_weights(codes, sbytes):
    """Values of one orientation [E][X][Y] (blocks along Y)."""
    return np.stack([dequant_mx_rows(codes[e], sbytes[e]) for e in range(codes.shape[0])])


def quant_mx_token_blocks(X, offsets):
    """Weight-gradient operand X [P][C] (rows grouped by expert as `offsets`
    gives them): in every column, each expert's rows are cut into blocks of
    32 consecutive rows starting at the expert's first row (the last block
    short) and every block gets its own scale.

    Returns codes [P][C] (row r stays row r) and scale bytes [NB][C], where
    NB = sum_e ceil(m_e / 32) and block b of expert e is row
    token_block_offsets(offsets, 32)[e] + b.  A short block is quantised as
    its rows alone (absent rows contribute nothing to its amax)."""
    X = np.asarray(X, dtype=np.float32)
    P, C = X.shape
    b32 = token_block_offsets(offsets, MX_BLOCK)
    codes = np.zeros((P, C), dtype=np.uint8)
    sb = np.full((int(b32[-1]), C), 127, dtype=np.uint8)
    for e in range(len(offsets) - 1):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        for b, s in enumerate(range(r0, r1, MX_BLOCK)):
            t = min(s + MX_BLOCK, r1)
            seg = np.zeros((C, MX_BLOCK), dtype=np.float32)    # absent rows are zero
            seg[:, :t - s] = X[s:t].T
            c_blk, s_blk = _mx_groups(seg)                     # one block per column
            codes[s:t] = c_blk[:, :t - s].T
            sb[int(b32[e]) + b] = s_blk
    return codes, sb


def dequant_mx_token_blocks(codes, sb, offsets):
    """Values [P][C] of the token-block operand (codes [P][C], bytes [NB][C])."""
    vals = e4m3_decode(codes)
    out = np.zeros_like(vals)
    b32 = token_block_offsets(offsets, MX_BLOCK)
    for e in range(len(offsets) - 1):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        for b, s in enumerate(range(r0, r1, MX_BLOCK)):
            t = min(s + MX_BLOCK, r1)
            out[s:t] = vals[s:t] * _scale_values(sb[int(b32[e]) + b])[None, :]
    return out


def _segments(offsets):
    for e in range(len(offsets) - 1):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 > r0:
            yield e, slice(r0, r1)


def fc1_fwd_mx(xpq, xps, offsets, W1td, W3td):
    """a = xp W1, b = xp W3 from the quantised rows of xp and the dequantised
    column-blocked weights W1td, W3td [E][f][d] (transposed orientation)."""
    X = dequant_mx_rows(xpq, xps)
    P, f = X.shape[0], W1td.shape[1]
    a = np.zeros((P, f)); b = np.zeros((P, f))
    for e, R in _segments(offsets):
        a[R] = X[R] @ W1td[e].T
        b[R] = X[R] @ W3td[e].T
    return a, b


def fc2_fwd_mx(h, offsets, W2td):
    """o = Q(h) W2; h quantised in 1 x 32 blocks along f, W2td [E][d][f]."""
    H = dequant_mx_rows(*quant_mx_rows(h))
    o = np.zeros((H.shape[0], W2td.shape[1]))
    for e, R in _segments(offsets):
        o[R] = H[R] @ W2td[e].T
    return o


def fc2_dgrad_mx(dO, a, b, offsets, W2d):
    """dH = Q(dO) W2^T with the row-blocked W2d [E][f][d], then the SwiGLU
    backward on the unquantised a, b."""
    G = dequant_mx_rows(*quant_mx_rows(dO))
    a = np.asarray(a, np.float64); b = np.asarray(b, np.float64)
    dH = np.zeros_like(a)
    for e, R in _segments(offsets):
        dH[R] = G[R] @ W2d[e].T
    s = sigmoid(a)
    return dH * b * s * (1.0 + a * (1.0 - s)), dH * silu(a)


def fc1_dgrad_mx(dab, offsets, W1d, W3d):
    """dXp = Q([da|db]) [W1|W3]^T with the row-blocked W1d, W3d [E][d][f]."""
    D = dequant_mx_rows(*quant_mx_rows(dab))
    f = W1d.shape[2]
    dXp = np.zeros((D.shape[0], W1d.shape[1]))
    for e, R in _segments(offsets):
        dXp[R] = D[R, :f] @ W1d[e].T + D[R, f:] @ W3d[e].T
    return dXp


def wgrad_mx(A, B, offsets):
    """dW_e = Q(A_e)^T Q(B_e), both in 32-row token blocks per column."""
    Ad = dequant_mx_token_blocks(*quant_mx_token_blocks(A, offsets), offsets)
    Bd = dequant_mx_token_blocks(*quant_mx_token_blocks(B, offsets), offsets)
    E = len(offsets) - 1
    dW = np.zeros((E, Ad.shape[1], Bd.shape[1]))
    for e, R in _segments(offsets):
        dW[e] = Ad[R].T @ Bd[R]
    return dW


def layer_fwd_mx(logits, x, W1, W3, W2, k):
    """Route, quantise x rows, permute codes and scales, MXFP8 experts,
    combine, on the oracle's own intermediates (fp32 masters W1, W3, W2)."""
    E = W1.shape[0]
    idx, p = route(logits, k)
    counts, offsets, row_of, token_of = permute_map(idx, E)
    xq, xs = quant_mx_rows(x)
    xpq, xps = xq[token_of], xs[token_of]
    Wq = {n: quant_mx_weights(W) for n, W in (("W1", W1), ("W3", W3), ("W2", W2))}
    rowd = {n: dequant_mx_weights(q[0], q[1]) for n, q in Wq.items()}
    cold = {n: dequant_mx_weights(q[2], q[3]) for n, q in Wq.items()}
    a, b = fc1_fwd_mx(xpq, xps, offsets, cold["W1"], cold["W3"])
    h = silu(a) * b
    o = fc2_fwd_mx(h, offsets, cold["W2"])
    return dict(idx=idx, p=p, counts=counts, offsets=offsets, row_of=row_of, token_of=token_of,
                xq=xq, xs=xs, xpq=xpq, xps=xps, a=a, b=b, h=h, o=o, rowd=rowd, cold=cold,
                y=combine(o, row_of, p))


def layer_bwd_mx(st, x, dY):
    """Backward of layer_fwd_mx: dO = p dY permuted, MXFP8 data and weight
    gradients, dX = un-permuted sum of dXp."""
    dO = permute_scaled(np.asarray(dY, np.float64), st["row_of"], st["p"])
    off = st["offsets"]
    da, db = fc2_dgrad_mx(dO, st["a"], st["b"], off, st["rowd"]["W2"])
    dab = np.concatenate([da, db], axis=1)
    dXp = fc1_dgrad_mx(dab, off, st["rowd"]["W1"], st["rowd"]["W3"])
    dW2 = wgrad_mx(st["h"], dO, off)
    xp = np.asarray(x, np.float64)[st["token_of"]]
    dW13 = wgrad_mx(xp, dab, off)
    f = st["a"].shape[1]
    return dict(dO=dO, da=da, db=db, dXp=dXp, dW2=dW2, dW1=dW13[:, :, :f], dW3=dW13[:, :, f:],
                dX=combine(dXp, st["row_of"]))
