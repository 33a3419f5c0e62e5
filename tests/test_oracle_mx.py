"""Pins of the MXFP8 oracle (oracle/mx.py), CPU only.

* the scale exponent against brute force over s and at its boundaries;
* codes: lossless on inputs built on the grid (every 32-value block holds
  e4m3 values times 2^s with its largest magnitude in (224, 448] * 2^s),
  within half an e4m3 step of the block scale otherwise, never saturated;
* layouts: both weight orientations and the per-expert token-block layout against
  a per-block construction by hand;
* products: on grid inputs whose block exponents differ from block to block,
  every MXFP8 product equals the plain fp64 product of oracle/moe.py exactly,
  so a scale taken from the wrong block, orientation or token block fails;
* the whole MXFP8 chain stays close to the unquantised layer.
"""
import numpy as np
import pytest

import oracle
from oracle.e4m3 import e4m3_decode, token_block_offsets
from oracle.mx import (dequant_mx_rows, dequant_mx_token_blocks, dequant_mx_weights,
                       mx_scale_exp, quant_mx_rows, quant_mx_token_blocks, quant_mx_weights)

RNG = np.random.default_rng(32)


def brute_exp(a):
    if a == 0:
        return 0
    for s in range(-127, 128):
        if a <= 448.0 * 2.0 ** s:
            return s
    raise AssertionError


def test_scale_exponent_boundaries():
    cases = {448.0: 0, 224.0: -1, 225.0: 0, 1.0: -8, 1.75: -8, 1.7500001: -7, 0.0: 0,
             float(np.nextafter(np.float32(448), np.float32(1e9))): 1,
             2.0 ** -140: -127, 3.0e38: 120, 448.0 * 2 ** 100: 100}
    for a, s in cases.items():
        assert int(mx_scale_exp(np.float32(a))) == s, a


def test_scale_exponent_brute_force():
    a = np.concatenate([np.exp(RNG.uniform(-90, 88, 3000)),
                        448.0 * 2.0 ** RNG.integers(-60, 60, 200)]).astype(np.float32)
    got = mx_scale_exp(a)
    for x, s in zip(a, got):
        assert s == brute_exp(float(x))


def grid_blocks(shape, rng, smin=-8, smax=4):
    """Values lossless in 1 x 32 blocks along the last axis: e4m3 grid values
    times 2^s per block, each block's largest magnitude in (224, 448] * 2^s."""
    *lead, K = shape
    c = rng.integers(0, 0x7E, size=shape)
    c = np.where(rng.random(shape) < 0.5, c, c | 0x80).astype(np.uint8)
    V = e4m3_decode(c)
    nb = K // 32
    top = rng.integers(0x77, 0x7F, size=(*lead, nb))       # 240 .. 448
    top = e4m3_decode(top.astype(np.uint8)) * np.where(rng.random((*lead, nb)) < 0.5, 1, -1)
    V = V.reshape(*lead, nb, 32)
    V[..., 0] = top
    s = rng.integers(smin, smax, size=(*lead, nb)).astype(np.float64)
    return (V * (2.0 ** s)[..., None]).reshape(shape), s


def test_rows_lossless_on_grid():
    X, s = grid_blocks((40, 256), RNG)
    q, sb = quant_mx_rows(X)
    assert np.array_equal(sb.astype(np.int64) - 127, s.astype(np.int64))
    assert np.array_equal(dequant_mx_rows(q, sb), X)


def test_rows_error_bound_and_no_saturation():
    X = (RNG.standard_normal((64, 512)) * np.exp(RNG.uniform(-6, 6, (64, 1)))).astype(np.float32)
    X[3, :32] = 0.0
    X[4, 32:64] = -0.0
    q, sb = quant_mx_rows(X)
    assert (q[3, :32] == 0).all() and (q[4, 32:64] == 0).all()
    assert sb[3, 0] == 127 and sb[4, 1] == 127
    vals = e4m3_decode(q)
    assert np.abs(vals).max() <= 448.0
    blockmax = np.abs(vals).reshape(64, 16, 32).max(-1)
    assert (blockmax[np.abs(X).reshape(64, 16, 32).max(-1) > 0] > 224.0 * 0.99).all()
    D = dequant_mx_rows(q, sb)
    scale = np.repeat(np.ldexp(1.0, sb.astype(np.int64) - 127), 32, axis=1)
    # half a step of the e4m3 grid: 2^-4 relative for normals, 2^-10 * scale below 2^-6
    bound = np.maximum(np.abs(X) * 2.0 ** -4, 2.0 ** -10 * scale)
    assert (np.abs(D - X) <= bound * (1 + 1e-12)).all()


def test_weight_orientations():
    E, R, C = 2, 64, 96
    # rows of very different magnitude: row blocks and column blocks get different scales
    W = (RNG.standard_normal((E, R, C)) * 2.0 ** RNG.integers(-6, 6, (E, R, 1))).astype(np.float32)
    q, sb, qt, sbt = quant_mx_weights(W)
    assert q.shape == (E, R, C) and sb.shape == (E, R, C // 32)
    assert qt.shape == (E, C, R) and sbt.shape == (E, C, R // 32)
    for e in range(E):
        for r in range(0, R, 7):
            for b in range(C // 32):
                c1, s1 = quant_mx_rows(W[e, r:r + 1, 32 * b:32 * b + 32])
                assert np.array_equal(q[e, r, 32 * b:32 * b + 32], c1[0]) and sb[e, r, b] == s1[0, 0]
        for c in range(0, C, 5):
            for b in range(R // 32):
                c1, s1 = quant_mx_rows(W[e, 32 * b:32 * b + 32, c][None, :])
                assert np.array_equal(qt[e, c, 32 * b:32 * b + 32], c1[0])
                assert sbt[e, c, b] == s1[0, 0]
    # orientations differ in general: blocks along rows vs along columns
    assert not np.array_equal(dequant_mx_weights(q, sb), dequant_mx_weights(qt, sbt).transpose(0, 2, 1))


def small_offsets():
    m = np.array([100, 0, 128, 33, 1])
    return np.concatenate([[0], np.cumsum(m)]).astype(np.int64)


def test_token_block_layout():
    """Each 32-row block of each expert, per column, is quantised alone:
    compare with quant_mx_rows on the block's values, built here by slicing."""
    off = small_offsets()
    P, C = int(off[-1]), 64
    X = np.random.default_rng(7).standard_normal((P, C)).astype(np.float32)
    X[100:132, 5] = 0.0                                      # an all-zero block (expert 2's first)
    X[224:228] *= 1000.0                                     # expert 2's last rows: large values
    q, sb = quant_mx_token_blocks(X, off)
    b32 = token_block_offsets(off, 32)
    assert q.shape == (P, C) and sb.shape == (int(b32[-1]), C)
    assert list(b32) == [0, 4, 4, 8, 10, 11]                 # ceil(m_e / 32) = 4, 0, 4, 2, 1
    for e in range(len(off) - 1):
        r0, r1 = int(off[e]), int(off[e + 1])
        for g, s in enumerate(range(r0, r1, 32)):
            t = min(s + 32, r1)
            for c in (0, 5, 17, 63):
                seg = np.zeros(32, np.float32)
                seg[:t - s] = X[s:t, c]
                c1, s1 = quant_mx_rows(seg[None, :])
                assert sb[int(b32[e]) + g, c] == s1[0, 0]
                assert np.array_equal(q[s:t, c], c1[0, :t - s])
    assert sb[4, 5] == 127 and not q[100:132, 5].any()       # zero block: s = 0, +0 codes
    D = dequant_mx_token_blocks(q, sb, off)
    assert np.abs(D - X).max() <= np.abs(X).max() * 2.0 ** -4
    # blocks restart at each expert: expert 3 (rows 228..260) has blocks
    # 228..259 and 260, not the fixed-stride blocks 224..255 and 256..287
    # (whose scales the large rows 224..227 of expert 2 would raise)
    assert off[3] == 228 and off[4] == 261
    alt_q, alt_s = quant_mx_rows(np.ascontiguousarray(X[224:256].T))
    assert not (np.array_equal(sb[8], alt_s[:, 0]) and np.array_equal(q[228:256], alt_q.T[4:]))


def grid_token_operand(P, C, off, rng):
    """[P][C] lossless in 32-row blocks per column inside every expert."""
    V = np.zeros((P, C))
    for e in range(len(off) - 1):
        r0, r1 = int(off[e]), int(off[e + 1])
        for r in range(r0, r1, 32):
            t = min(r + 32, r1)
            blkv, _ = grid_blocks((C, 32), rng, -5, 3)
            V[r:t] = blkv[:, :t - r].T
            # keep the block's maximum inside the rows that exist
            V[r, :] = blkv[:, 0]
    return V


def test_products_exact_on_grid():
    """Every MXFP8 product equals the fp64 product when its inputs are lossless."""
    rng = np.random.default_rng(7)
    E, d, f = 3, 64, 96
    off = np.array([0, 45, 45, 110]).astype(np.int64)          # expert 1 empty
    P = int(off[-1])
    # weights lossless in both orientations: one value per 32 x 32 tile scale
    base = e4m3_decode(rng.integers(0, 0x7E, size=(E, d, f)).astype(np.uint8))
    base[:, ::32, ::32] = 448.0
    st = rng.integers(-9, -3, size=(E, d // 32, f // 32)).astype(np.float64)
    W = base * np.repeat(np.repeat(2.0 ** st, 32, axis=1), 32, axis=2)
    q, sb, qt, sbt = quant_mx_weights(W)
    Wr, Wc = dequant_mx_weights(q, sb), dequant_mx_weights(qt, sbt)
    assert np.array_equal(Wr, W) and np.array_equal(Wc.transpose(0, 2, 1), W)
    X, _ = grid_blocks((P, d), rng)
    xq, xs = quant_mx_rows(X)
    a, b = oracle.fc1_fwd_mx(xq, xs, off, Wc, Wc)
    for e in range(E):
        R = slice(int(off[e]), int(off[e + 1]))
        assert np.array_equal(a[R], X[R] @ W[e])
        assert np.array_equal(b[R], X[R] @ W[e])
    H, _ = grid_blocks((P, f), rng)
    W2 = np.ascontiguousarray(W.transpose(0, 2, 1))                 # [E][f][d]
    q2, sb2, qt2, sbt2 = quant_mx_weights(W2)
    o = oracle.fc2_fwd_mx(H, off, dequant_mx_weights(qt2, sbt2))
    G, _ = grid_blocks((P, d), rng)
    aa, bb = rng.standard_normal((P, f)), rng.standard_normal((P, f))
    da, db = oracle.fc2_dgrad_mx(G, aa, bb, off, dequant_mx_weights(q2, sb2))
    D, _ = grid_blocks((P, 2 * f), rng)
    dXp = oracle.fc1_dgrad_mx(D, off, Wr, Wr)
    for e in range(E):
        R = slice(int(off[e]), int(off[e + 1]))
        assert np.array_equal(o[R], H[R] @ W2[e])
        dH = G[R] @ W2[e].T
        s = oracle.sigmoid(aa[R])
        assert np.allclose(da[R], dH * bb[R] * s * (1 + aa[R] * (1 - s)), rtol=0, atol=1e-12)
        assert np.array_equal(dXp[R], D[R, :f] @ W[e].T + D[R, f:] @ W[e].T)
    A = grid_token_operand(P, d, off, rng)
    B = grid_token_operand(P, f, off, rng)
    dW = oracle.wgrad_mx(A, B, off)
    for e in range(E):
        R = slice(int(off[e]), int(off[e + 1]))
        assert np.array_equal(dW[e], A[R].T @ B[R])
    assert not dW[1].any()


def test_chain_close_to_unquantised_layer():
    rng = np.random.default_rng(3)
    T, d, E, k, f = 96, 128, 4, 2, 128
    L = rng.standard_normal((T, E)).astype(np.float32)
    x = rng.standard_normal((T, d)).astype(np.float32)
    W1 = (rng.standard_normal((E, d, f)) * d ** -0.5).astype(np.float32)
    W3 = (rng.standard_normal((E, d, f)) * d ** -0.5).astype(np.float32)
    W2 = (rng.standard_normal((E, f, d)) * f ** -0.5).astype(np.float32)
    dY = rng.standard_normal((T, d)).astype(np.float32)
    st = oracle.layer_fwd_mx(L, x, W1, W3, W2, k)
    g = oracle.layer_bwd_mx(st, x, dY)
    ref = oracle.layer_fwd(L, x, W1, W3, W2, k)
    rg = oracle.layer_bwd(ref, dY, W1, W3, W2)
    # the same bounds as the blockwise e4m3 chain's (3 mantissa bits per element)
    assert oracle.row_rel_err(st["y"], ref["y"]) < 0.2
    assert oracle.row_rel_err(g["dX"], rg["dX"]) < 0.2
    for n in ("dW1", "dW3", "dW2"):
        assert oracle.row_rel_err(g[n], rg[n]) < 0.3, n
    # and it is a different chain from the blockwise e4m3 one
    st8 = oracle.layer_fwd_e4m3(L, x, W1, W3, W2, k)
    assert not np.array_equal(st8["y"], st["y"])


def test_layer_forward_uses_column_blocked_weights():
    """Weights lossless only in 32 x 1 column blocks (the scale changes from
    column to column inside a row block): the forward products, which contract
    over the weights' rows, must be exact, so they must use that orientation."""
    rng = np.random.default_rng(11)
    T, d, E, k, f = 64, 64, 2, 1, 64
    base = e4m3_decode(rng.integers(0, 0x7E, size=(E, d, f)).astype(np.uint8))
    base[:, ::32, :] = 448.0
    s = rng.integers(-9, -2, size=(E, d // 32, f)).astype(np.float64)
    W = base * np.repeat(2.0 ** s, 32, axis=1)
    q, sb, qt, sbt = quant_mx_weights(W)
    assert np.array_equal(dequant_mx_weights(qt, sbt).transpose(0, 2, 1), W)
    assert not np.array_equal(dequant_mx_weights(q, sb), W)
    x, _ = grid_blocks((T, d), rng)
    L = rng.standard_normal((T, E)).astype(np.float32)
    st = oracle.layer_fwd_mx(L, x, W, W, W, k)
    xp = x[st["token_of"]]
    for e in range(E):
        R = slice(int(st["offsets"][e]), int(st["offsets"][e + 1]))
        assert np.array_equal(st["a"][R], xp[R] @ W[e])
