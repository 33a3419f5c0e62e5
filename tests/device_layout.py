"""Index maps between the device's storage layouts and the oracle's plain ones.

Data movement only (slicing and reshaping, no arithmetic): the oracle states
every quantised operand in the operand's own shape, while the library stores
the weight-gradient operands in the layout its kernels read.  These helpers
take a device buffer apart so that the tests can compare it with the oracle
element by element, and check that the device's padding holds what the
library's header promises.

Device token-block scales (include/moe.h, moe_quantize_token_blocks_mx):
with blk128 = first 128-row block of each expert (prefix sum of
ceil(m_e / 128)), MXFP8 scale bytes are [cap][C][4], byte g of (block b,
column c) scaling rows 32 g .. 32 g + 31 of block b (the codes are the
operand's own [P][C] rows and need no map).
"""
from __future__ import annotations

import numpy as np


def _blocks(offsets, rows_per_block):
    offsets = np.asarray(offsets, dtype=np.int64)
    nb = (np.diff(offsets) + rows_per_block - 1) // rows_per_block
    return np.concatenate([[0], np.cumsum(nb)]).astype(np.int64)


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
