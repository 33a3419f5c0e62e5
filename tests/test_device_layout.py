"""CPU checks of tests/device_layout.py: the index maps invert a device layout
built here cell by cell from the header's description."""
import numpy as np
import pytest

import device_layout


def _device_from_logical(sb32, offsets, cap, C):
    """Build the device token-block scale layout cell by cell (the header's
    description, written as loops)."""
    sbw = np.full((cap, C, 4), 127, np.uint8)
    blk128 = 0
    blk32 = 0
    for e in range(len(offsets) - 1):
        m = int(offsets[e + 1] - offsets[e])
        for g in range((m + 31) // 32):
            b, slot = blk128 + g // 4, g % 4
            sbw[b, :, slot] = sb32[blk32 + g]
        blk128 += (m + 127) // 128
        blk32 += (m + 31) // 32
    return sbw


def test_token_block_scale_map_inverts_the_device_layout():
    rng = np.random.default_rng(5)
    m = [130, 0, 31, 128, 1, 64]
    off = np.concatenate([[0], np.cumsum(m)]).astype(np.int64)
    C = 7
    nb32 = sum((x + 31) // 32 for x in m)
    sb32 = rng.integers(100, 126, size=(nb32, C)).astype(np.uint8)
    cap = sum((x + 127) // 128 for x in m) + 2                 # unused blocks at the end
    sbw = _device_from_logical(sb32, off, cap, C)
    assert np.array_equal(device_layout.mx_token_block_scales(sbw, off), sb32)
    # a wrong padding byte is reported
    bads = sbw.copy()
    bads[2, 0, 1] = 120                                        # expert 2: one 32-row block, slot 1 unused
    with pytest.raises(AssertionError):
        device_layout.mx_token_block_scales(bads, off)
