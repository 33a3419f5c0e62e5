"""fp64 oracle of route -> permute -> SwiGLU experts -> combine, and its backward.

TEST INFRASTRUCTURE ONLY (see the package docstring).

All floating-point work is float64 on exactly up-cast inputs.  Citations name
the page ("Scalable Training of Mixture-of-Experts Models with Megatron Core",
gist.science summary in the stated language) and its section.

Shapes: T tokens, d hidden, E experts, k experts per token, f FFN width,
P = T*k routed rows.  Weights: W1, W3 are [E][d][f], W2 is [E][f][d] (each
expert maps d -> f -> d).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "route", "permute_map", "permute_rows", "permute_scaled", "silu", "sigmoid",
    "swiglu_fwd", "swiglu_bwd", "experts_fwd", "experts_bwd", "combine",
    "layer_fwd", "layer_bwd", "token_fwd_bwd", "expert_wgrad", "row_rel_err",
]


# ---------------------------------------------------------------- routing
def route(logits: np.ndarray, k: int):
    """Top-k routing from router logits.

    Follows the Spanish technical summary, section 2.1 (a router sends each
    token to its k best experts).  The pages do not say how the k weights are
    formed; the reading used here is a softmax over the k selected logits.

    Per token t the experts are fully sorted by the key (-logit, expert index)
    with a stable sort, so equal logits (IEEE equality, -0 == +0) keep the
    lower expert index first; the first k form idx[t].  Selection compares the
    stored fp32 logits.  A NaN logit sorts after every number (-inf included;
    NaNs among themselves by index), which is NumPy's ordering of NaN, so the
    k picks are always k distinct experts.  Then, with m the largest selected
    logit, p[t, j] = exp(l_j - m) / sum_i exp(l_i - m), all in fp64 (NaN for
    every pick of a token that has a NaN among its picks).

    Returns idx int32 [T][k] (descending logit, lower index first on ties)
    and p float64 [T][k].
    """
    L = np.asarray(logits, dtype=np.float64)
    T, E = L.shape
    assert 1 <= k <= E
    order = np.argsort(-L, axis=1, kind="stable")
    idx = order[:, :k]
    sel = np.take_along_axis(L, idx, axis=1)
    m = sel[:, :1]
    ex = np.exp(sel - m)
    p = ex / ex.sum(axis=1, keepdims=True)
    return idx.astype(np.int32), p


# ---------------------------------------------------------------- permutation
def permute_map(idx: np.ndarray, E: int):
    """Dropless token -> expert-contiguous row map.

    Follows the Spanish technical summary, section 2.1 (dispatch moves each
    token to the location of its assigned experts) and the German technical
    summary, section 1 (dropless routing: every assignment is computed, with
    dynamic per-expert sizes).  On one GPU dispatch is a local reordering.

    counts[e] = number of (t, j) with idx[t, j] == e; offsets is its exclusive
    prefix sum with offsets[E] = T*k.  The canonical order is a stable sort of
    the token-major flattened idx: within an expert, rows ascend by token.
    row_of[t, j] is the row of assignment (t, j); token_of[r] the token of row r.
    """
    T, k = idx.shape
    flat = idx.reshape(-1).astype(np.int64)
    counts = np.bincount(flat, minlength=E).astype(np.int64)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    order = np.argsort(flat, kind="stable")
    row_of = np.empty(T * k, dtype=np.int64)
    row_of[order] = np.arange(T * k)
    token_of = order // k
    return counts, offsets, row_of.reshape(T, k), token_of


def permute_rows(x: np.ndarray, token_of: np.ndarray) -> np.ndarray:
    """xp[r] = x[token_of[r]]: a plain row copy (values unchanged)."""
    return x[token_of]


def permute_scaled(dY: np.ndarray, row_of: np.ndarray, p: np.ndarray) -> np.ndarray:
    """Backward of the weighted combine: dO[row_of[t, j]] = p[t, j] * dY[t]."""
    T, k = row_of.shape
    dO = np.zeros((T * k, dY.shape[1]), dtype=np.float64)
    for j in range(k):
        dO[row_of[:, j]] = p[:, j:j + 1] * dY
    return dO


# ---------------------------------------------------------------- experts
def sigmoid(z):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def silu(z):
    """SiLU with beta = 1: z * sigmoid(z) = z / (1 + e^-z)."""
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_fwd(X, W1, W3, W2):
    """One SwiGLU expert: a = X W1, b = X W3, h = silu(a) * b, o = h W2.

    The pages do not name the expert FFN; the reading used is SwiGLU with the
    gate on W1 and the linear branch on W3.
    """
    a = X @ W1
    b = X @ W3
    h = silu(a) * b
    return a, b, h, h @ W2


def swiglu_bwd(X, a, b, h, dO, W1, W3, W2):
    """Backward of swiglu_fwd for upstream gradient dO (rows of X).

    dW2 = h^T dO; dH = dO W2^T; with s = sigmoid(a):
    da = dH * b * s * (1 + a (1 - s)) (derivative of silu), db = dH * silu(a);
    dX = da W1^T + db W3^T; dW1 = X^T da; dW3 = X^T db.
    """
    dW2 = h.T @ dO
    dH = dO @ W2.T
    s = sigmoid(a)
    da = dH * b * s * (1.0 + a * (1.0 - s))
    db = dH * silu(a)
    dX = da @ W1.T + db @ W3.T
    return dX, X.T @ da, X.T @ db, dW2, da, db


def experts_fwd(xp, offsets, W1, W3, W2):
    """Per-expert SwiGLU on the expert-contiguous rows (the grouped GEMM).

    Follows the Spanish technical summary, section 2.1 (compute: local expert
    execution by grouped GEMM) and section 2.3 C (one grouped GEMM bundles the
    small expert GEMMs).  Experts with no rows contribute nothing.
    """
    P, d = xp.shape
    E, _, f = W1.shape
    a = np.zeros((P, f)); b = np.zeros((P, f)); h = np.zeros((P, f)); o = np.zeros((P, d))
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 > r0:
            a[r0:r1], b[r0:r1], h[r0:r1], o[r0:r1] = swiglu_fwd(xp[r0:r1], W1[e], W3[e], W2[e])
    return a, b, h, o


def experts_bwd(dO, xp, a, b, h, offsets, W1, W3, W2):
    """Per-expert backward: data gradient dXp and weight gradients dW1, dW3, dW2.

    The data- and weight-gradient products are separate, as in the German
    technical summary, section 2 C (W/D split).  An expert with no rows gets
    exactly zero weight gradients.
    """
    E, d, f = W1.shape
    dXp = np.zeros_like(xp, dtype=np.float64)
    dW1 = np.zeros((E, d, f)); dW3 = np.zeros((E, d, f)); dW2 = np.zeros((E, f, d))
    da = np.zeros_like(a); db = np.zeros_like(b)
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 > r0:
            R = slice(r0, r1)
            dXp[R], dW1[e], dW3[e], dW2[e], da[R], db[R] = swiglu_bwd(
                xp[R], a[R], b[R], h[R], dO[R], W1[e], W3[e], W2[e])
    return dXp, dW1, dW3, dW2, da, db


# ---------------------------------------------------------------- combine
def combine(src, row_of, p=None, add=None):
    """Weighted un-permute: y[t] = sum_j p[t, j] * src[row_of[t, j]] (+ add[t]).

    Follows the Spanish technical summary, section 2.1 (combine returns the
    processed tokens to their origin).  p = None means weight 1 (the backward
    of permute: dX[t] = sum_j dXp[row_of[t, j]]).  The sum runs j = 0..k-1.
    """
    T, k = row_of.shape
    y = np.zeros((T, src.shape[1]))
    for j in range(k):
        w = 1.0 if p is None else p[:, j:j + 1]
        y += w * src[row_of[:, j]]
    if add is not None:
        y += add
    return y


# ---------------------------------------------------------------- whole layer
def layer_fwd(logits, x, W1, W3, W2, k, shared=None):
    """Forward of the layer: route, permute, experts, combine (+ shared expert).

    `shared` = (Ws1, Ws3, Ws2) adds a SwiGLU expert applied to every token with
    weight 1 (DeepSeek-V3-class layers; not on the pages, which name the model
    only).  Returns a dict of every intermediate, all float64.
    """
    E = W1.shape[0]
    x = np.asarray(x, dtype=np.float64)
    idx, p = route(logits, k)
    counts, offsets, row_of, token_of = permute_map(idx, E)
    xp = permute_rows(x, token_of)
    a, b, h, o = experts_fwd(xp, offsets, W1, W3, W2)
    st = dict(idx=idx, p=p, counts=counts, offsets=offsets, row_of=row_of, token_of=token_of,
              xp=xp, a=a, b=b, h=h, o=o, x=x)
    ys = None
    if shared is not None:
        sa, sb, sh, ys = swiglu_fwd(x, *shared)
        st.update(sa=sa, sb=sb, sh=sh, ys=ys)
    st["y"] = combine(o, row_of, p, ys)
    return st


def layer_bwd(st, dY, W1, W3, W2, shared=None):
    """Backward of layer_fwd for upstream gradient dY.

    The logits are an input of the layer, so no gradient flows to them or to
    the routing weights; the outputs are dX, dW1, dW3, dW2 (and the shared
    expert's dWs1, dWs3, dWs2).
    """
    dY = np.asarray(dY, dtype=np.float64)
    dO = permute_scaled(dY, st["row_of"], st["p"])
    dXp, dW1, dW3, dW2, da, db = experts_bwd(dO, st["xp"], st["a"], st["b"], st["h"],
                                              st["offsets"], W1, W3, W2)
    g = dict(dO=dO, dXp=dXp, dW1=dW1, dW3=dW3, dW2=dW2, da=da, db=db)
    dXs = None
    if shared is not None:
        dXs, dWs1, dWs3, dWs2, _, _ = swiglu_bwd(st["x"], st["sa"], st["sb"], st["sh"], dY, *shared)
        g.update(dWs1=dWs1, dWs3=dWs3, dWs2=dWs2, dXs=dXs)
    g["dX"] = combine(dXp, st["row_of"], None, dXs)
    return g


# ---------------------------------------------------------------- sampled forms
def token_fwd_bwd(x_t, dY_t, idx_t, p_t, W1, W3, W2, shared=None):
    """y[t] and dX[t] for one token, from its own routing row only.

    The same definitions as layer_fwd/layer_bwd restricted to one token: every
    term of y[t] and dX[t] depends on row t alone, so this equals the full
    oracle's rows exactly (up to rounding order).
    """
    x_t = np.asarray(x_t, dtype=np.float64)[None, :]
    dY_t = np.asarray(dY_t, dtype=np.float64)[None, :]
    y = np.zeros_like(x_t); dX = np.zeros_like(x_t)
    for j in range(len(idx_t)):
        e = int(idx_t[j])
        a, b, h, o = swiglu_fwd(x_t, W1[e], W3[e], W2[e])
        y += p_t[j] * o
        dXj, *_ = swiglu_bwd(x_t, a, b, h, p_t[j] * dY_t, W1[e], W3[e], W2[e])
        dX += dXj
    if shared is not None:
        a, b, h, ys = swiglu_fwd(x_t, *shared)
        y += ys
        dXs, *_ = swiglu_bwd(x_t, a, b, h, dY_t, *shared)
        dX += dXs
    return y[0], dX[0]


def expert_wgrad(X_e, dO_e, W1_e, W3_e, W2_e):
    """Weight gradients of one expert from its rows X_e and their upstream
    gradients dO_e (already multiplied by the routing weights)."""
    X_e = np.asarray(X_e, dtype=np.float64)
    a, b, h, _ = swiglu_fwd(X_e, W1_e, W3_e, W2_e)
    _, dW1, dW3, dW2, _, _ = swiglu_bwd(X_e, a, b, h, np.asarray(dO_e, np.float64), W1_e, W3_e, W2_e)
    return dW1, dW3, dW2


# ---------------------------------------------------------------- parity metric
def row_rel_err(got, ref) -> float:
    """max over rows of max_i |got - ref| / max_i |ref|.

    A reference row that is all zero requires the other row to be exactly
    zero (error 0 if so, +inf otherwise).
    """
    g = np.asarray(got, dtype=np.float64).reshape(-1, np.shape(ref)[-1])
    r = np.asarray(ref, dtype=np.float64).reshape(-1, np.shape(ref)[-1])
    den = np.abs(r).max(axis=1)
    num = np.abs(g - r).max(axis=1)
    err = np.where(den > 0, num / np.where(den > 0, den, 1.0), np.where(num > 0, np.inf, 0.0))
    return float(err.max()) if err.size else 0.0
