"""Pins of the e4m3 expert-GEMM oracle (oracle/moe_e4m3.py), CPU only.

Inputs built exactly on the e4m3 grid -- every quantisation block holds
e4m3-representable values times 2^s with its largest magnitude exactly
448 * 2^s -- quantise without loss (scale = 2^s, codes exact), so each e4m3
product must equal the plain fp64 product of oracle/moe.py exactly.  The block
exponents s differ from block to block, so a scale taken from the wrong block
(a transposed tile grid, a row/column mix-up, a wrong token-block start) fails.
Random inputs check the quantisation error against its bound.
"""
import numpy as np
import pytest

import oracle
from oracle.e4m3 import e4m3_decode, quant_rows, quant_tiles, token_block_offsets

RNG = np.random.default_rng(20261202)
MAXC = 0x7E  # code of 448


def grid_values(shape, rng):
    """e4m3-representable values (no NaN codes), random signs."""
    c = rng.integers(0, 0x7E, size=shape)
    c = np.where(rng.random(shape) < 0.5, c, c | 0x80)
    return e4m3_decode(c.astype(np.uint8))


def grid_rows(R, K, rng):
    """[R][K] with 1 x 128 blocks lossless: block (r, b) = grid * 2^s(r, b)."""
    V = grid_values((R, K), rng)
    V[:, ::128] = 448.0 * np.where(rng.random((R, K // 128)) < 0.5, 1.0, -1.0)
    s = rng.integers(-6, 4, size=(R, K // 128)).astype(np.float64)
    return V * np.repeat(2.0 ** s, 128, axis=1)


def grid_tiles(E, R, C, rng):
    """[E][R][C] with 128 x 128 tiles lossless."""
    V = grid_values((E, R, C), rng)
    V[:, ::128, ::128] = 448.0
    s = rng.integers(-9, -2, size=(E, R // 128, C // 128)).astype(np.float64)
    return V * np.repeat(np.repeat(2.0 ** s, 128, axis=1), 128, axis=2)


def grid_token_blocks(P, C, offsets, rng):
    """[P][C] with per-expert 128-row blocks lossless in every column."""
    V = grid_values((P, C), rng)
    for e in range(len(offsets) - 1):
        for r in range(int(offsets[e]), int(offsets[e + 1]), 128):
            V[r, :] = 448.0 * np.where(rng.random(C) < 0.5, 1.0, -1.0)
            s = rng.integers(-5, 3, size=C).astype(np.float64)
            t = min(r + 128, int(offsets[e + 1]))
            V[r:t] *= 2.0 ** s[None, :]
    return V


def small_offsets():
    # 4 experts: 300 rows (3 blocks, short last), 0 rows, 128 rows, 77 rows
    m = np.array([300, 0, 128, 77])
    return np.concatenate([[0], np.cumsum(m)]).astype(np.int64)


def test_grid_inputs_quantise_losslessly():
    X = grid_rows(5, 256, RNG)
    q, s = quant_rows(X)
    assert np.array_equal(oracle.dequant_rows(q, s), X)
    W = grid_tiles(1, 256, 384, RNG)[0]
    q, s = quant_tiles(W)
    assert np.array_equal(oracle.dequant_tiles(q, s), W)


def test_fc1_fwd_equals_plain_product_on_grid():
    off = small_offsets(); P = int(off[-1]); E, d, f = 4, 256, 384
    X = grid_rows(P, d, RNG)
    W1 = grid_tiles(E, d, f, RNG); W3 = grid_tiles(E, d, f, RNG); W2 = grid_tiles(E, f, d, RNG)
    xq, xs = quant_rows(X)
    W1d = oracle.dequant_expert_weights(*oracle.quant_expert_weights(W1))
    W3d = oracle.dequant_expert_weights(*oracle.quant_expert_weights(W3))
    assert np.array_equal(W1d, W1) and np.array_equal(W3d, W3)
    a, b = oracle.fc1_fwd_e4m3(xq, xs, off, W1d, W3d)
    ra, rb, _, _ = oracle.experts_fwd(X, off, W1, W3, W2)
    assert np.array_equal(a, ra) and np.array_equal(b, rb)


def test_fc2_fwd_and_dgrads_equal_plain_products_on_grid():
    off = small_offsets(); P = int(off[-1]); E, d, f = 4, 256, 384
    W1 = grid_tiles(E, d, f, RNG); W3 = grid_tiles(E, d, f, RNG); W2 = grid_tiles(E, f, d, RNG)
    W2d = oracle.dequant_expert_weights(*oracle.quant_expert_weights(W2))
    assert np.array_equal(W2d, W2)
    H = grid_rows(P, f, RNG)
    o = oracle.fc2_fwd_e4m3(H, off, W2d)
    ref = np.zeros((P, d))
    for e in range(E):
        R = slice(int(off[e]), int(off[e + 1]))
        ref[R] = H[R] @ W2[e]
    assert np.array_equal(o, ref)
    # fc2 dgrad + SwiGLU backward == experts_bwd's da, db for the same a, b, dO
    X = RNG.standard_normal((P, d)); dO = grid_rows(P, d, RNG)
    a, b, h, _ = oracle.experts_fwd(X, off, W1, W3, W2)
    _, _, _, _, rda, rdb = oracle.experts_bwd(dO, X, a, b, h, off, W1, W3, W2)
    da, db = oracle.fc2_dgrad_e4m3(dO, a, b, off, W2d)
    assert np.allclose(da, rda, rtol=1e-12, atol=1e-300) and np.allclose(db, rdb, rtol=1e-12, atol=1e-300)
    # fc1 dgrad on grid [da|db]
    D = grid_rows(P, 2 * f, RNG)
    dXp = oracle.fc1_dgrad_e4m3(D, off, W1, W3)
    ref = np.zeros((P, d))
    for e in range(E):
        R = slice(int(off[e]), int(off[e + 1]))
        ref[R] = D[R, :f] @ W1[e].T + D[R, f:] @ W3[e].T
    assert np.allclose(dXp, ref, rtol=1e-13, atol=0)


def test_wgrad_equals_plain_product_on_token_block_grid():
    off = small_offsets(); P = int(off[-1])
    A = grid_token_blocks(P, 256, off, RNG)
    B = grid_token_blocks(P, 384, off, RNG)
    dW = oracle.wgrad_e4m3(A, B, off)
    for e in range(4):
        R = slice(int(off[e]), int(off[e + 1]))
        assert np.allclose(dW[e], A[R].T @ B[R], rtol=1e-13, atol=0)
    assert not dW[1].any()  # the empty expert
    assert token_block_offsets(off).tolist() == [0, 3, 3, 4, 5]


def test_products_stay_within_quantisation_error_on_random_inputs():
    """Normal inputs: each operand is off by at most 1/16 relative (3 mantissa
    bits, round to nearest), so a product's row error normalised by the row
    max stays far below 0.25; a wrong scale gives errors of order 1."""
    off = small_offsets(); P = int(off[-1]); E, d, f = 4, 256, 384
    X = RNG.standard_normal((P, d)) * np.exp(RNG.standard_normal((P, 1)))
    W1 = RNG.standard_normal((E, d, f)) / 16; W3 = RNG.standard_normal((E, d, f)) / 16
    W2 = RNG.standard_normal((E, f, d)) / 20
    xq, xs = quant_rows(X)
    W1d = oracle.dequant_expert_weights(*oracle.quant_expert_weights(W1))
    W3d = oracle.dequant_expert_weights(*oracle.quant_expert_weights(W3))
    a, b = oracle.fc1_fwd_e4m3(xq, xs, off, W1d, W3d)
    ra, rb, rh, ro = oracle.experts_fwd(X, off, W1, W3, W2)
    assert oracle.row_rel_err(a, ra) < 0.25 and oracle.row_rel_err(b, rb) < 0.25
    W2d = oracle.dequant_expert_weights(*oracle.quant_expert_weights(W2))
    assert oracle.row_rel_err(oracle.fc2_fwd_e4m3(rh, off, W2d), ro) < 0.25
    dW = oracle.wgrad_e4m3(X, rh, off)
    for e in (0, 2, 3):
        R = slice(int(off[e]), int(off[e + 1]))
        assert oracle.row_rel_err(dW[e], X[R].T @ rh[R]) < 0.25


def test_layer_chain_close_to_unquantised_layer():
    T, d, E, k, f = 96, 128, 4, 2, 256
    logits = RNG.standard_normal((T, E)).astype(np.float32)
    x = RNG.standard_normal((T, d)).astype(np.float32)
    W1 = (RNG.standard_normal((E, d, f)) / np.sqrt(d)).astype(np.float32)
    W3 = (RNG.standard_normal((E, d, f)) / np.sqrt(d)).astype(np.float32)
    W2 = (RNG.standard_normal((E, f, d)) / np.sqrt(f)).astype(np.float32)
    dY = RNG.standard_normal((T, d)).astype(np.float32)
    st = oracle.layer_fwd_e4m3(logits, x, W1, W3, W2, k)
    g = oracle.layer_bwd_e4m3(st, x, dY)
    rs = oracle.layer_fwd(logits, x, W1.astype(np.float64), W3.astype(np.float64),
                          W2.astype(np.float64), k)
    rg = oracle.layer_bwd(rs, dY, W1.astype(np.float64), W3.astype(np.float64),
                          W2.astype(np.float64))
    assert np.array_equal(st["row_of"], rs["row_of"])
    assert oracle.row_rel_err(st["y"], rs["y"]) < 0.2
    assert oracle.row_rel_err(g["dX"], rg["dX"]) < 0.2
    for n in ("dW1", "dW3", "dW2"):
        assert oracle.row_rel_err(g[n], rg[n]) < 0.3, n
