"""Pins of the oracle's SwiGLU experts, combine and backward.

Independent references: torch autograd on a per-token loop (a different
derivation of every gradient), central finite differences, closed forms and
algebraic invariants.
"""
import numpy as np
import pytest
import torch

import oracle


def make(T, d, E, k, f, seed=0, fs=0):
    rng = np.random.default_rng(seed)
    L = rng.standard_normal((T, E)).astype(np.float32)
    x = rng.standard_normal((T, d))
    W1 = rng.standard_normal((E, d, f)) / np.sqrt(d)
    W3 = rng.standard_normal((E, d, f)) / np.sqrt(d)
    W2 = rng.standard_normal((E, f, d)) / np.sqrt(f)
    dY = rng.standard_normal((T, d))
    shared = None
    if fs:
        shared = (rng.standard_normal((d, fs)) / np.sqrt(d), rng.standard_normal((d, fs)) / np.sqrt(d),
                  rng.standard_normal((fs, d)) / np.sqrt(fs))
    return L, x, W1, W3, W2, dY, shared


def torch_layer(L, x, W1, W3, W2, dY, k, shared=None):
    """Per-token autograd reference: y[t] = sum_j p_tj * FFN_e(x_t)."""
    tx = torch.tensor(x, requires_grad=True)
    tw = [torch.tensor(w, requires_grad=True) for w in (W1, W3, W2)]
    ts = [torch.tensor(w, requires_grad=True) for w in shared] if shared is not None else None
    Lt = torch.tensor(L, dtype=torch.float64)
    rows = []
    for t in range(x.shape[0]):
        order = sorted(range(L.shape[1]), key=lambda e: (-float(L[t, e]), e))[:k]
        p = torch.softmax(Lt[t, order], 0)
        yt = 0
        for j, e in enumerate(order):
            h = torch.nn.functional.silu(tx[t] @ tw[0][e]) * (tx[t] @ tw[1][e])
            yt = yt + p[j] * (h @ tw[2][e])
        if ts is not None:
            yt = yt + (torch.nn.functional.silu(tx[t] @ ts[0]) * (tx[t] @ ts[1])) @ ts[2]
        rows.append(yt)
    y = torch.stack(rows)
    (y * torch.tensor(dY)).sum().backward()
    out = dict(y=y.detach().numpy(), dX=tx.grad.numpy(), dW1=tw[0].grad.numpy(),
               dW3=tw[1].grad.numpy(), dW2=tw[2].grad.numpy())
    if ts is not None:
        out.update(dWs1=ts[0].grad.numpy(), dWs3=ts[1].grad.numpy(), dWs2=ts[2].grad.numpy())
    return out


@pytest.mark.parametrize("T,d,E,k,f,fs", [(24, 8, 4, 2, 6, 0), (17, 6, 5, 3, 4, 5), (10, 4, 3, 3, 5, 0)])
def test_layer_matches_torch_autograd(T, d, E, k, f, fs):
    L, x, W1, W3, W2, dY, shared = make(T, d, E, k, f, seed=T, fs=fs)
    st = oracle.layer_fwd(L, x, W1, W3, W2, k, shared)
    g = oracle.layer_bwd(st, dY, W1, W3, W2, shared)
    ref = torch_layer(L, x, W1, W3, W2, dY, k, shared)
    assert np.allclose(st["y"], ref["y"], rtol=1e-12, atol=1e-12)
    for name in ("dX", "dW1", "dW3", "dW2") + (("dWs1", "dWs3", "dWs2") if fs else ()):
        assert np.allclose(g[name], ref[name], rtol=1e-11, atol=1e-12), name


def test_finite_differences_micro_layer():
    T, d, E, k, f = 8, 4, 4, 2, 6
    L, x, W1, W3, W2, dY, _ = make(T, d, E, k, f, seed=11)
    st = oracle.layer_fwd(L, x, W1, W3, W2, k)
    g = oracle.layer_bwd(st, dY, W1, W3, W2)

    def loss(x_, W1_, W3_, W2_):
        return float((oracle.layer_fwd(L, x_, W1_, W3_, W2_, k)["y"] * dY).sum())

    rng = np.random.default_rng(0)
    eps = 1e-6
    for name, arr, grad in (("x", x, g["dX"]), ("W1", W1, g["dW1"]), ("W3", W3, g["dW3"]),
                            ("W2", W2, g["dW2"])):
        for _ in range(6):
            pos = tuple(rng.integers(0, s) for s in arr.shape)
            args = {"x": x, "W1": W1, "W3": W3, "W2": W2}
            plus = {n: a.copy() for n, a in args.items()}
            minus = {n: a.copy() for n, a in args.items()}
            plus[name][pos] += eps
            minus[name][pos] -= eps
            num = (loss(plus["x"], plus["W1"], plus["W3"], plus["W2"]) -
                   loss(minus["x"], minus["W1"], minus["W3"], minus["W2"])) / (2 * eps)
            assert abs(num - grad[pos]) <= 1e-6 * max(1.0, abs(num)), (name, pos, num, grad[pos])


def test_empty_expert_has_zero_weight_grad():
    T, d, E, k, f = 30, 6, 5, 2, 4
    L, x, W1, W3, W2, dY, _ = make(T, d, E, k, f, seed=2)
    L[:, 3] -= 100.0                                   # expert 3 is never selected
    st = oracle.layer_fwd(L, x, W1, W3, W2, k)
    g = oracle.layer_bwd(st, dY, W1, W3, W2)
    assert st["counts"][3] == 0
    assert (g["dW1"][3] == 0).all() and (g["dW3"][3] == 0).all() and (g["dW2"][3] == 0).all()
    assert np.abs(g["dW1"][0]).sum() > 0


def test_scaling_W2():
    T, d, E, k, f = 20, 5, 4, 2, 7
    L, x, W1, W3, W2, dY, _ = make(T, d, E, k, f, seed=3)
    alpha = 2.5
    st = oracle.layer_fwd(L, x, W1, W3, W2, k)
    g = oracle.layer_bwd(st, dY, W1, W3, W2)
    st2 = oracle.layer_fwd(L, x, W1, W3, alpha * W2, k)
    g2 = oracle.layer_bwd(st2, dY, W1, W3, alpha * W2)
    assert np.allclose(st2["y"], alpha * st["y"], rtol=1e-13, atol=1e-13)
    for n in ("dX", "dW1", "dW3"):
        assert np.allclose(g2[n], alpha * g[n], rtol=1e-12, atol=1e-13), n
    assert np.allclose(g2["dW2"], g["dW2"], rtol=1e-13, atol=1e-14)


def test_single_expert_is_dense_swiglu():
    T, d, f = 9, 7, 5
    L, x, W1, W3, W2, dY, _ = make(T, d, 1, 1, f, seed=4)
    st = oracle.layer_fwd(L, x, W1, W3, W2, 1)
    assert (st["p"] == 1.0).all()
    tx = torch.tensor(x)
    ref = (torch.nn.functional.silu(tx @ torch.tensor(W1[0])) * (tx @ torch.tensor(W3[0]))) @ torch.tensor(W2[0])
    assert np.allclose(st["y"], ref.numpy(), rtol=1e-13, atol=1e-13)


def test_silu_against_torch_and_closed_forms():
    z = np.linspace(-30, 30, 601)
    assert np.allclose(oracle.silu(z), torch.nn.functional.silu(torch.tensor(z)).numpy(), rtol=1e-14, atol=1e-300)
    assert oracle.silu(0.0) == 0.0
    assert np.isclose(oracle.silu(1.0), 1.0 / (1.0 + np.exp(-1.0)), rtol=1e-15)
    assert np.isclose(oracle.silu(-10.0), -10.0 * np.exp(-10.0) / (1.0 + np.exp(-10.0)), rtol=1e-14)
    assert np.allclose(oracle.sigmoid(z), torch.sigmoid(torch.tensor(z)).numpy(), rtol=1e-14)


def test_token_order_covariance():
    T, d, E, k, f = 25, 6, 6, 2, 5
    L, x, W1, W3, W2, dY, _ = make(T, d, E, k, f, seed=6)
    perm = np.random.default_rng(1).permutation(T)
    st = oracle.layer_fwd(L, x, W1, W3, W2, k)
    g = oracle.layer_bwd(st, dY, W1, W3, W2)
    st2 = oracle.layer_fwd(L[perm], x[perm], W1, W3, W2, k)
    g2 = oracle.layer_bwd(st2, dY[perm], W1, W3, W2)
    assert np.allclose(st2["y"], st["y"][perm], rtol=1e-13, atol=1e-14)
    assert np.allclose(g2["dX"], g["dX"][perm], rtol=1e-13, atol=1e-14)
    for n in ("dW1", "dW3", "dW2"):
        assert np.allclose(g2[n], g[n], rtol=1e-12, atol=1e-13), n


def test_shared_expert_only():
    T, d, E, k, f, fs = 12, 5, 4, 2, 3, 6
    L, x, W1, W3, W2, dY, shared = make(T, d, E, k, f, seed=7, fs=fs)
    st = oracle.layer_fwd(L, x, W1, W3, np.zeros_like(W2), k, shared)
    tx = torch.tensor(x)
    ref = (torch.nn.functional.silu(tx @ torch.tensor(shared[0])) * (tx @ torch.tensor(shared[1]))) @ torch.tensor(shared[2])
    assert np.allclose(st["y"], ref.numpy(), rtol=1e-13, atol=1e-13)


def test_sampled_forms_equal_full_layer():
    T, d, E, k, f, fs = 40, 8, 6, 3, 5, 4
    L, x, W1, W3, W2, dY, shared = make(T, d, E, k, f, seed=8, fs=fs)
    st = oracle.layer_fwd(L, x, W1, W3, W2, k, shared)
    g = oracle.layer_bwd(st, dY, W1, W3, W2, shared)
    for t in (0, 7, 39):
        y_t, dX_t = oracle.token_fwd_bwd(x[t], dY[t], st["idx"][t], st["p"][t], W1, W3, W2, shared)
        assert np.allclose(y_t, st["y"][t], rtol=1e-13, atol=1e-14)
        assert np.allclose(dX_t, g["dX"][t], rtol=1e-13, atol=1e-14)
    for e in range(E):
        R = slice(st["offsets"][e], st["offsets"][e + 1])
        dW1, dW3, dW2 = oracle.expert_wgrad(st["xp"][R], g["dO"][R], W1[e], W3[e], W2[e])
        assert np.allclose(dW1, g["dW1"][e], atol=1e-13) and np.allclose(dW3, g["dW3"][e], atol=1e-13)
        assert np.allclose(dW2, g["dW2"][e], atol=1e-13)
