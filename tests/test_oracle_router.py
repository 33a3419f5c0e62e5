"""Pins of the router-backward and auxiliary-loss oracle (oracle/router.py), CPU only.

Independent derivations: torch autograd of the top-k softmax combine and of the
load-balancing loss written out in torch; central finite differences; the
closed form L = alpha for equal logits (every P_e = 1/E and sum_e f_e = 1).
"""
import numpy as np
import pytest
import torch

import oracle

RNG = np.random.default_rng(99)


def _case(T=37, E=9, k=3, d=11):
    L = RNG.standard_normal((T, E))
    idx, p = oracle.route(L.astype(np.float32), k)
    counts, offsets, row_of, token_of = oracle.permute_map(idx, E)
    o = RNG.standard_normal((T * k, d))
    dY = RNG.standard_normal((T, d))
    return L, idx, p, counts, row_of, o, dY


def test_router_bwd_matches_autograd():
    L, idx, p, counts, row_of, o, dY = _case()
    T, E = L.shape
    k = idx.shape[1]
    Lt = torch.tensor(L.astype(np.float32).astype(np.float64), requires_grad=True)
    sel = Lt.gather(1, torch.from_numpy(idx.astype(np.int64)))
    pt = torch.softmax(sel, dim=1)
    O = torch.from_numpy(o)[torch.from_numpy(row_of.astype(np.int64))]      # [T][k][d]
    y = (pt[:, :, None] * O).sum(dim=1)
    (y * torch.from_numpy(dY)).sum().backward()
    dp = oracle.combine_dprob(dY, o, row_of)
    got = oracle.router_bwd(dp, p, idx, E)
    assert np.allclose(got, Lt.grad.numpy(), rtol=1e-5, atol=1e-9)
    # unselected experts get exactly zero
    mask = np.zeros((T, E), bool)
    mask[np.arange(T)[:, None], idx] = True
    assert not got[~mask].any()


def test_combine_dprob_is_the_probability_gradient():
    L, idx, p, counts, row_of, o, dY = _case(T=5, E=6, k=2, d=4)
    pt = torch.tensor(p.astype(np.float64), requires_grad=True)
    O = torch.from_numpy(o)[torch.from_numpy(row_of.astype(np.int64))]
    y = (pt[:, :, None] * O).sum(dim=1)
    (y * torch.from_numpy(dY)).sum().backward()
    assert np.allclose(oracle.combine_dprob(dY, o, row_of), pt.grad.numpy(), rtol=1e-12)


def test_aux_loss_matches_autograd_and_closed_form():
    L, idx, p, counts, row_of, o, dY = _case(T=50, E=8, k=2)
    T, E = L.shape
    alpha = 0.01
    loss, dL = oracle.aux_loss(L, counts, 2, alpha)
    Lt = torch.tensor(L, requires_grad=True)
    s = torch.softmax(Lt, dim=1)
    f = torch.from_numpy(counts.astype(np.float64)) / (T * 2)
    ref = alpha * E * (f * s.mean(dim=0)).sum()
    ref.backward()
    assert abs(loss - ref.item()) <= 1e-12 * abs(ref.item())
    assert np.allclose(dL, Lt.grad.numpy(), rtol=1e-9, atol=1e-15)
    # equal logits: P_e = 1/E for every e and sum_e f_e = 1, so L = alpha; and the gradient vanishes
    # only where f is uniform -- check the value
    Lz = np.zeros((T, E))
    lz, _ = oracle.aux_loss(Lz, counts, 2, alpha)
    assert abs(lz - alpha) <= 1e-15


def test_router_and_aux_by_finite_differences():
    T, E, k, d = 6, 5, 2, 3
    L = RNG.standard_normal((T, E))
    idx, p = oracle.route(L.astype(np.float32), k)
    counts, offsets, row_of, token_of = oracle.permute_map(idx, E)
    o = RNG.standard_normal((T * k, d))
    dY = RNG.standard_normal((T, d))

    def total(Lm):
        # selection kept fixed (it is piecewise constant); p recomputed from the logits
        sel = np.take_along_axis(Lm, idx, axis=1)
        q = np.exp(sel - sel.max(axis=1, keepdims=True))
        q /= q.sum(axis=1, keepdims=True)
        y = sum(q[:, j:j + 1] * o[row_of[:, j]] for j in range(k))
        return float(np.sum(y * dY)) + oracle.aux_loss(Lm, counts, k, 0.1)[0]

    dp = oracle.combine_dprob(dY, o, row_of)
    p64 = np.take_along_axis(L, idx, axis=1)
    p64 = np.exp(p64 - p64.max(axis=1, keepdims=True)); p64 /= p64.sum(axis=1, keepdims=True)
    g = oracle.router_bwd(dp, p64, idx, E) + oracle.aux_loss(L, counts, k, 0.1)[1]
    h = 1e-6
    fd = np.zeros_like(L)
    for t in range(T):
        for e in range(E):
            Lp = L.copy(); Lp[t, e] += h
            Lm = L.copy(); Lm[t, e] -= h
            fd[t, e] = (total(Lp) - total(Lm)) / (2 * h)
    assert np.allclose(g, fd, rtol=1e-6, atol=1e-8)
