"""CPU checks of tests/device_layout.py: the index maps invert a device layout
built here cell by cell from the header's description."""
import numpy as np
import pytest

import device_layout


def _device_from_logical(q, sb32, offsets, cap):
    """Build the device token-block layout cell by cell (the header's
    description, written as loops)."""
    P, C = q.shape
    codes_t = np.zeros((C, 128 * cap), np.uint8)
    sbw = np.full((cap, C, 4), 127, np.uint8)
    blk128 = 0
    blk32 = 0
    for e in range(len(offsets) - 1):
        m = int(offsets[e + 1] - offsets[e])
        for i in range(m):
            r = int(offsets[e]) + i
            codes_t[:, 128 * blk128 + i] = q[r]
        for g in range((m + 31) // 32):
            b, slot = blk128 + g // 4, g % 4
            sbw[b, :, slot] = sb32[blk32 + g]
        blk128 += (m + 127) // 128
        blk32 += (m + 31) // 32
    return codes_t, sbw


def test_token_block_maps_invert_the_device_layout():
    rng = np.random.default_rng(5)
    m = [130, 0, 31, 128, 1, 64]
    off = np.concatenate([[0], np.cumsum(m)]).astype(np.int64)
    P, C = int(off[-1]), 7
    q = rng.integers(1, 255, size=(P, C)).astype(np.uint8)
    nb32 = sum((x + 31) // 32 for x in m)
    sb32 = rng.integers(100, 126, size=(nb32, C)).astype(np.uint8)
    cap = sum((x + 127) // 128 for x in m) + 2                 # unused blocks at the end
    codes_t, sbw = _device_from_logical(q, sb32, off, cap)
    assert np.array_equal(device_layout.token_block_codes(codes_t, off), q)
    assert np.array_equal(device_layout.mx_token_block_scales(sbw, off), sb32)
    # a non-zero padding code or a wrong padding byte is reported
    bad = codes_t.copy()
    bad[3, 128 * 1 + 2] = 9                                    # expert 0's second block, column 130
    with pytest.raises(AssertionError):
        device_layout.token_block_codes(bad, off)
    bads = sbw.copy()
    bads[2, 0, 1] = 120                                        # expert 2: one 32-row block, slot 1 unused
    with pytest.raises(AssertionError):
        device_layout.mx_token_block_scales(bads, off)
