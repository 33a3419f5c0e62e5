"""Pins of the oracle's routing and permutation against brute force and invariants."""
import numpy as np
import pytest
import scipy.special
import torch

import oracle
from moe_workloads import tied_logits


def brute_topk(row, k):
    """k rounds of argmax, pure Python: strictly larger wins, so the first
    (lowest) index wins among equal values."""
    taken = set()
    out = []
    for _ in range(k):
        best = None
        for e, v in enumerate(row):
            if e in taken:
                continue
            if best is None or v > row[best]:
                best = e
        taken.add(best)
        out.append(best)
    return out


@pytest.mark.parametrize("T,E,k,tied", [(16, 8, 2, False), (16, 8, 2, True), (9, 16, 4, True),
                                        (7, 5, 5, True), (11, 6, 1, True), (5, 64, 8, False)])
def test_route_matches_k_round_argmax(T, E, k, tied):
    L = (tied_logits(T, E, levels=3, seed=T * E) if tied
         else torch.randn(T, E, generator=torch.Generator().manual_seed(1))).numpy()
    idx, p = oracle.route(L, k)
    for t in range(T):
        assert list(idx[t]) == brute_topk([float(v) for v in L[t]], k)
        sel = [float(L[t, e]) for e in idx[t]]
        m = max(sel)
        ex = [np.exp(v - m) for v in sel]
        assert np.allclose(p[t], [v / sum(ex) for v in ex], rtol=0, atol=1e-15)


def brute_topk_nan_last(row, k):
    """k rounds of a pure-Python scan in which a NaN ranks below every
    number (-inf included) and equal keys keep the lower index."""
    def key(e):
        v = row[e]
        return (0, 0.0) if v != v else (1, v)
    taken, out = set(), []
    for _ in range(k):
        best = None
        for e in range(len(row)):
            if e not in taken and (best is None or key(e) > key(best)):
                best = e
        taken.add(best)
        out.append(best)
    return out


def test_route_nan_ranks_last():
    nan, inf = float("nan"), float("inf")
    L = np.array([[nan, 1.0, nan, -inf, 0.5, nan],
                  [nan, nan, nan, nan, nan, nan],
                  [-inf, nan, -inf, 2.0, nan, -inf],
                  [0.0, -0.0, nan, 3.0, -inf, 1.0]], dtype=np.float32)
    for k in (1, 3, 4, 6):
        idx, p = oracle.route(L, k)
        for t in range(L.shape[0]):
            assert list(idx[t]) == brute_topk_nan_last([float(v) for v in L[t]], k)
            assert len(set(idx[t])) == k and (idx[t] >= 0).all() and (idx[t] < 6).all()
            picked = L[t, idx[t]]
            if np.isnan(picked).any():
                assert np.isnan(p[t]).all()
            else:
                assert np.isfinite(p[t]).all() or np.isinf(picked[0])
    idx, p = oracle.route(L, 3)
    assert list(idx[0]) == [1, 4, 3] and list(idx[1]) == [0, 1, 2] and list(idx[2]) == [3, 0, 2]


def test_route_all_equal_logits():
    for k in (1, 2, 3, 8):
        L = np.full((4, 8), 0.75, dtype=np.float32)
        idx, p = oracle.route(L, k)
        assert (idx == np.arange(k)[None, :]).all()
        assert (p == 1.0 / k).all()


def test_route_signed_zero_is_a_tie():
    L = np.array([[-0.0, 0.0, -1.0, 0.0]], dtype=np.float32)
    idx, _ = oracle.route(L, 3)
    assert list(idx[0]) == [0, 1, 3]


def test_route_k_equals_E_is_full_softmax():
    L = np.random.default_rng(3).standard_normal((10, 7)).astype(np.float32)
    idx, p = oracle.route(L, 7)
    full = scipy.special.softmax(L.astype(np.float64), axis=1)
    assert np.allclose(p, np.take_along_axis(full, idx, 1), rtol=0, atol=1e-15)


def test_route_prob_invariants():
    L = np.random.default_rng(4).standard_normal((200, 32)).astype(np.float32)
    idx, p = oracle.route(L, 6)
    assert np.allclose(p.sum(1), 1.0, atol=1e-15)
    assert (np.diff(p, axis=1) <= 0).all()
    sel = np.take_along_axis(L, idx, 1)
    assert (np.diff(sel, axis=1) <= 0).all()
    for t in range(200):                         # selected are the k largest
        assert sel[t].min() >= np.delete(L[t], idx[t]).max()


def brute_permute(idx, E):
    T, k = idx.shape
    row_of = -np.ones((T, k), dtype=np.int64)
    token_of = []
    counts = [0] * E
    for e in range(E):
        for t in range(T):
            for j in range(k):
                if idx[t, j] == e:
                    row_of[t, j] = len(token_of)
                    token_of.append(t)
                    counts[e] += 1
    return np.array(counts), row_of, np.array(token_of)


@pytest.mark.parametrize("T,E,k", [(12, 4, 2), (33, 8, 3), (5, 5, 5), (40, 16, 1), (1, 3, 2)])
def test_permute_matches_brute_force(T, E, k):
    L = tied_logits(T, E, levels=4, seed=T + E).numpy()
    idx, _ = oracle.route(L, k)
    counts, offsets, row_of, token_of = oracle.permute_map(idx, E)
    bc, brow, btok = brute_permute(idx, E)
    assert (counts == bc).all() and (row_of == brow).all() and (token_of == btok).all()
    assert offsets[0] == 0 and offsets[-1] == T * k and (np.diff(offsets) == counts).all()


def test_permute_invariants_and_identity_experts():
    rng = np.random.default_rng(5)
    T, E, k, d = 300, 12, 3, 10
    L = rng.standard_normal((T, E)).astype(np.float32)
    x = rng.standard_normal((T, d))
    idx, p = oracle.route(L, k)
    counts, offsets, row_of, token_of = oracle.permute_map(idx, E)
    assert counts.sum() == T * k
    assert np.array_equal(np.sort(row_of.ravel()), np.arange(T * k))          # bijection
    assert (token_of[row_of] == np.arange(T)[:, None]).all()
    for e in range(E):                                                     # stable segments
        seg = token_of[offsets[e]:offsets[e + 1]]
        assert (np.diff(seg) > 0).all()
        assert (idx[seg] == e).any(axis=1).all()
    xp = oracle.permute_rows(x, token_of)
    assert (xp[row_of[:, 1]] == x).all()
    # identity experts (o = xp): the probabilities sum to one, so y = x
    y = oracle.combine(xp, row_of, p)
    assert np.allclose(y, x, rtol=1e-14, atol=1e-14)
    # unpermute with weights 1/k inverts permute
    assert np.allclose(oracle.combine(xp, row_of, np.full((T, k), 1.0 / k)), x, atol=1e-14)
    # permute_scaled is the adjoint of the weighted combine: <combine(o), dY> = <o, dO>
    o = rng.standard_normal((T * k, d))
    dY = rng.standard_normal((T, d))
    dO = oracle.permute_scaled(dY, row_of, p)
    assert np.isclose((oracle.combine(o, row_of, p) * dY).sum(), (o * dO).sum(), rtol=1e-12)


def test_row_rel_err_semantics():
    ref = np.array([[1.0, -2.0], [0.0, 0.0]])
    assert oracle.row_rel_err(ref, ref) == 0.0
    assert np.isclose(oracle.row_rel_err(ref + [[0.02, 0.0], [0, 0]], ref), 0.01)
    assert oracle.row_rel_err(ref + [[0, 0], [1e-30, 0]], ref) == np.inf
