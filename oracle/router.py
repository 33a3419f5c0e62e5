"""fp64 oracle of the router backward and the load-balancing auxiliary loss.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages fuse routing, permutation and auxiliary-loss computations into few
kernels ("Scalable Training of Mixture-of-Experts Models with Megatron Core",
gist.science German technical summary, section 2 D "Kernel Fusion"; Spanish
summary, section 2.3 C) but state no formula for either.  Readings used:

* router backward: the layer output is y[t] = sum_j p[t,j] o[row_of[t,j]]
  (+ the shared expert, which does not depend on the logits) with p the
  softmax over the k selected logits.  With dp[t,j] = <dY[t], o[row_of[t,j]]>
  the logit gradient is p_j (dp_j - sum_i p_i dp_i) on the k selected experts
  (the softmax Jacobian) and 0 on the others; the selection itself is piecewise
  constant and contributes nothing;
* auxiliary loss: the switch-style load-balancing loss
      L = alpha * E * sum_e f_e * P_e,
  f_e = counts_e / (T k), the share of routing slots that went to expert e, and
  P_e = (1/T) sum_t s[t,e], the mean over tokens of the full softmax s over all
  E logits.  The counts are a step function of the logits and are held
  constant, so dL/dlogits[t] = s[t] * (g - <g, s[t]>) with g_e = alpha E f_e / T.
"""
from __future__ import annotations

import numpy as np

__all__ = ["combine_dprob", "router_bwd", "aux_loss"]


def combine_dprob(dY, o, row_of):
    """dp[t, j] = <dY[t], o[row_of[t, j]]>: gradient of the weighted combine
    with respect to the routing probabilities."""
    dY = np.asarray(dY, np.float64)
    o = np.asarray(o, np.float64)
    T, k = row_of.shape
    dp = np.zeros((T, k))
    for j in range(k):
        dp[:, j] = np.sum(dY * o[row_of[:, j]], axis=1)
    return dp


def router_bwd(dp, p, idx, E):
    """dlogits [T][E] of the top-k softmax: p_j (dp_j - sum_i p_i dp_i) at the
    selected experts idx[t, j], 0 elsewhere."""
    dp = np.asarray(dp, np.float64)
    p = np.asarray(p, np.float64)
    T, k = idx.shape
    inner = np.sum(p * dp, axis=1, keepdims=True)
    g = p * (dp - inner)
    dl = np.zeros((T, E))
    for j in range(k):
        dl[np.arange(T), idx[:, j]] += g[:, j]
    return dl


def aux_loss(logits, counts, k, alpha):
    """(L, dL/dlogits) of the switch-style load-balancing loss (module docstring)."""
    L = np.asarray(logits, np.float64)
    T, E = L.shape
    s = np.exp(L - L.max(axis=1, keepdims=True))
    s /= s.sum(axis=1, keepdims=True)
    f = np.asarray(counts, np.float64) / (T * k)
    P = s.mean(axis=0)
    loss = alpha * E * float(np.sum(f * P))
    g = alpha * E * f / T
    dL = s * (g[None, :] - (s @ g)[:, None])
    return loss, dL
