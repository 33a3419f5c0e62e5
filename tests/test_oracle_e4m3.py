"""Pins of the e4m3 block-quantisation oracle.

Independent references: torch's float8_e4m3fn dtype (decode of all 256
codes, and round-to-nearest-even encode inside its finite range), exact
round trips of blocks built on the e4m3 grid, and the half-ulp error bound.
"""
import numpy as np
import torch

import oracle
from oracle.e4m3 import E4M3_MAX


def torch_decode_all():
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_decode_table_matches_torch():
    ours = oracle.e4m3_value_table()
    ref = torch_decode_all()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))
    assert ours[0x7E] == E4M3_MAX and ours[0x01] == 2.0 ** -9


def test_encode_matches_torch_rne_in_range():
    vals = oracle.e4m3_value_table()[:127]
    mids = (vals[:-1] + vals[1:]) / 2                       # exact ties
    rng = np.random.default_rng(0)
    v = np.concatenate([vals, mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
                        rng.uniform(-460, 460, 20000), rng.standard_normal(20000) * 2.0 ** -7,
                        rng.uniform(448, 463.9, 100)]).astype(np.float32)
    v = np.concatenate([v, -v])
    ours = oracle.e4m3_encode(v)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_encode_saturates():
    v = np.array([464.0, 1000.0, 3.0e38, -500.0, -1e30], dtype=np.float32)
    assert list(oracle.e4m3_encode(v)) == [0x7E, 0x7E, 0x7E, 0xFE, 0xFE]


def test_zero_block_and_signed_zero():
    c, s = oracle.quant_block(np.zeros(128, np.float32))
    assert s == 1.0 and (c == 0).all()
    c, s = oracle.quant_block(np.full(128, -0.0, np.float32))   # amax == 0: every code is +0
    assert s == 1.0 and (c == 0).all()
    c, s = oracle.quant_block(np.array([-0.0, 1.0] + [0.0] * 126, np.float32))
    assert c[0] == 0x80 and c[1] == 0x7E and s == np.float32(1.0) / np.float32(448.0)


def test_grid_blocks_round_trip_exactly():
    rng = np.random.default_rng(1)
    table = oracle.e4m3_value_table()[:127]
    for n in (-6, 0, 3):
        v = rng.choice(table, size=(4, 128)) * rng.choice([-1, 1], size=(4, 128))
        v[:, 5] = 448.0                                     # amax = 448 -> scale 1
        v = (v * 2.0 ** n).astype(np.float32)
        codes, scales = oracle.quant_rows(v)
        assert (scales == np.float32(2.0 ** n)).all()
        assert np.array_equal(oracle.dequant_rows(codes, scales), v.astype(np.float64))


def test_error_bound_half_ulp():
    rng = np.random.default_rng(2)
    v = (rng.standard_normal((64, 256)) * np.exp(rng.uniform(-8, 8, (64, 1)))).astype(np.float32)
    codes, scales = oracle.quant_rows(v)
    deq = oracle.dequant_rows(codes, scales)
    s = np.repeat(scales.astype(np.float64), 128, axis=1)
    u = np.abs(v.astype(np.float64)) / s                     # magnitude on the e4m3 grid
    e = np.floor(np.log2(np.maximum(u, 2.0 ** -6)))          # binade (subnormals share 2^-6)
    bound = s * 2.0 ** (e - 4) * (1 + 1e-6) + np.abs(v) * 2.0 ** -23
    assert (np.abs(deq - v) <= bound).all()


def test_tiles_and_token_blocks_follow_the_block_rule():
    rng = np.random.default_rng(3)
    W = rng.standard_normal((256, 384)).astype(np.float32)
    codes, scales = oracle.quant_tiles(W)
    for i in range(2):
        for j in range(3):
            c, s = oracle.quant_block(W[128 * i:128 * (i + 1), 128 * j:128 * (j + 1)])
            assert s == scales[i, j] and np.array_equal(c, codes[128 * i:128 * (i + 1), 128 * j:128 * (j + 1)])
    offsets = np.array([0, 0, 300, 301, 301, 460])
    X = rng.standard_normal((460, 5)).astype(np.float32)
    codes, scales = oracle.quant_token_blocks(X, offsets)
    blk = oracle.token_block_offsets(offsets)
    assert list(blk) == [0, 0, 3, 4, 4, 6]
    c, s = oracle.quant_block(X[256:300, 2])                 # expert 1's short third block
    assert s == scales[2, 2] and np.array_equal(c, codes[256:300, 2])
    c, s = oracle.quant_block(X[300:301, 4])                 # expert 2's single row
    assert s == scales[3, 4] and np.array_equal(c, codes[300:301, 4])
    deq = oracle.dequant_token_blocks(codes, scales, offsets)
    assert np.abs(deq - X).max() <= np.abs(X).max() / 448.0 * 16


def test_quantise_then_permute_equals_permute_then_quantise():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((50, 256)).astype(np.float32)
    L = rng.standard_normal((50, 6)).astype(np.float32)
    idx, _ = oracle.route(L, 2)
    _, _, _, token_of = oracle.permute_map(idx, 6)
    c1, s1 = oracle.quant_rows(x)
    c2, s2 = oracle.quant_rows(oracle.permute_rows(x, token_of))
    assert np.array_equal(c1[token_of], c2) and np.array_equal(s1[token_of], s2)
