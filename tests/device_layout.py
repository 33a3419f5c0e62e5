"""Index maps between the device's storage layouts and the oracle's plain ones.

Data movement only (slicing and reshaping, no arithmetic): the oracle states
every quantised operand in the operand's own shape, while the library stores
the weight-gradient operands in the layout its kernels read.  These helpers
take a device buffer apart so that the tests can compare it with the oracle
element by element, and check that the device's padding holds what the
library's header promises.

Device token-block layout (include/moe.h, moe_quantize_token_blocks and
moe_quantize_token_blocks_mx): with blk128 = first 128-row block of each
expert (prefix sum of ceil(m_e / 128)), row r of expert e is column
128 * blk128[e] + (r - offsets[e]) of the transposed codes [C][128 cap];
columns past the expert's rows in its last block hold code 0.  e4m3 scales
are fp32 [cap][C], one per 128-row block; MXFP8 scale bytes are [cap][C][4],
byte g of (block b, column c) scaling rows 32 g .. 32 g + 31 of block b.
"""
from __future__ import annotations

import numpy as np


def _blocks(offsets, rows_per_block):
    offsets = np.asarray(offsets, dtype=np.int64)
    nb = (np.diff(offsets) + rows_per_block - 1) // rows_per_block
    return np.concatenate([[0], np.cumsum(nb)]).astype(np.int64)


def token_block_codes(codes_t, offsets):
    """Transposed device codes [C][128 cap] -> codes [P][C] in row order.
    Asserts that the columns past each expert's rows in its last 128-row
    block are zero."""
    codes_t = np.asarray(codes_t)
    offsets = np.asarray(offsets, dtype=np.int64)
    b128 = _blocks(offsets, 128)
    P, C = int(offsets[-1]), codes_t.shape[0]
    out = np.zeros((P, C), dtype=codes_t.dtype)
    for e in range(len(offsets) - 1):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        c0, c1 = 128 * int(b128[e]), 128 * int(b128[e + 1])
        out[r0:r1] = codes_t[:, c0:c0 + (r1 - r0)].T
        assert not codes_t[:, c0 + (r1 - r0):c1].any(), f"expert {e}: non-zero padding codes"
    return out


def mx_token_block_scales(sbw, offsets):
    """Device MXFP8 token-block scale bytes [cap][C][4] -> the oracle's
    [NB32][C] (block b of expert e at row prefix-sum-of-ceil(m/32)[e] + b).
    Asserts that the 32-row slots of an expert's last 128-row block that hold
    no rows carry byte 127 (2^0)."""
    sbw = np.asarray(sbw)
    offsets = np.asarray(offsets, dtype=np.int64)
    b128, b32 = _blocks(offsets, 128), _blocks(offsets, 32)
    C = sbw.shape[1]
    flat = sbw.transpose(1, 0, 2).reshape(C, -1)          # [C][32-row slot], slot = 4 b + g
    out = np.zeros((int(b32[-1]), C), dtype=sbw.dtype)
    for e in range(len(offsets) - 1):
        n32 = int(b32[e + 1] - b32[e])
        s0, s1 = 4 * int(b128[e]), 4 * int(b128[e + 1])
        out[int(b32[e]):int(b32[e + 1])] = flat[:, s0:s0 + n32].T
        assert (flat[:, s0 + n32:s1] == 127).all(), f"expert {e}: padding scale bytes"
    return out
