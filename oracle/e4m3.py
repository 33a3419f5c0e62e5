"""fp8 (OCP E4M3FN) block quantisation oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages say that expert GEMMs run in FP8 with a blockwise recipe on Hopper
while the router stays in higher precision (gist.science French technical
summary, section 2 E "Précision réduite"; German technical summary, section
2 E: fp8 weights straight from fp32 masters).  They give no formula; the
reading used here:

* format: OCP E4M3FN -- sign, 4 exponent bits (bias 7), 3 mantissa bits,
  subnormals kept, no infinities, S.1111.111 is NaN, largest finite 448;
* a block B of fp32 values: amax = max |v|; if amax == 0 the scale is 1 and
  every code is +0; otherwise scale = fp32(amax / 448) (IEEE fp32 division)
  and q = E4M3(fp32(v / scale)) rounded to nearest, ties to even, saturating
  at +-448; the sign of q is the sign bit of v / scale (so -0 and tiny
  negatives give the code 0x80);
* dequantised value: q * scale (exact in fp64);
* block shapes: 1 x 128 along the contraction axis for activation operands,
  128 x 128 tiles for weights, and for weight-gradient operands (contraction
  over tokens) 128-token blocks per column, restarting at every expert's
  first row with a short last block.
"""
from __future__ import annotations

import numpy as np

__all__ = ["E4M3_MAX", "e4m3_value_table", "e4m3_decode", "e4m3_encode", "quant_block",
           "quant_rows", "dequant_rows", "quant_tiles", "dequant_tiles",
           "quant_token_blocks", "dequant_token_blocks", "token_block_offsets"]

E4M3_MAX = 448.0


def e4m3_value_table() -> np.ndarray:
    """Value of every code 0..255 (NaN for the two NaN codes), from the bit fields."""
    vals = np.empty(256, dtype=np.float64)
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        ex = (c >> 3) & 0xF
        m = c & 0x7
        if ex == 0xF and m == 0x7:
            vals[c] = np.nan
        elif ex == 0:
            vals[c] = s * (m / 8.0) * 2.0 ** -6
        else:
            vals[c] = s * (1.0 + m / 8.0) * 2.0 ** (ex - 7)
    return vals


_TABLE = e4m3_value_table()
_POS = _TABLE[:127]          # codes 0x00..0x7E: 0 .. 448, strictly increasing


def e4m3_decode(codes) -> np.ndarray:
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(v) -> np.ndarray:
    """Round fp32 values to the nearest E4M3FN code, ties to even, saturating.

    Brute force on the value table: the two neighbouring representable
    magnitudes are found by search; the closer one wins, and on an exact tie
    the one with the even code (even mantissa) wins.  |v| >= 448 gives 448.
    """
    v = np.asarray(v, dtype=np.float32)
    mag = np.abs(v.astype(np.float64))
    neg = np.signbit(v)
    hi = np.searchsorted(_POS, mag, side="left")          # first value >= mag
    hi = np.clip(hi, 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    dlo = mag - _POS[lo]
    dhi = _POS[hi] - mag
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(mag >= E4M3_MAX, 126, code)
    code = np.where(mag <= _POS[0], 0, code)
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)


def _quant_groups(V):
    """Quantise every vector along the last axis of V as one block.

    Returns codes uint8 (shape of V) and scales fp32 (V.shape[:-1]).
    """
    V = np.asarray(V, dtype=np.float32)
    amax = np.max(np.abs(V), axis=-1) if V.shape[-1] else np.zeros(V.shape[:-1], np.float32)
    zero = amax == 0
    scale = np.where(zero, np.float32(1.0), amax / np.float32(E4M3_MAX)).astype(np.float32)
    codes = e4m3_encode(V / scale[..., None])
    codes[zero] = 0
    return codes, scale


def quant_block(v):
    """Quantise one block of fp32 values -> (codes uint8, scale fp32)."""
    v = np.asarray(v, dtype=np.float32)
    codes, scale = _quant_groups(v.reshape(1, -1))
    return codes.reshape(v.shape), np.float32(scale[0])


def quant_rows(A, block: int = 128):
    """1 x `block` blocks along the last axis: codes [R][K], scales fp32 [R][K/block]."""
    A = np.asarray(A, dtype=np.float32)
    R, K = A.shape
    assert K % block == 0
    codes, scales = _quant_groups(A.reshape(R, K // block, block))
    return codes.reshape(R, K), scales


def dequant_rows(codes, scales, block: int = 128):
    vals = e4m3_decode(codes)
    return vals * np.repeat(np.asarray(scales, np.float64), block, axis=1)


def quant_tiles(W, block: int = 128):
    """`block` x `block` tiles of a 2-D matrix: codes [A][B], scales fp32 [A/block][B/block]."""
    W = np.asarray(W, dtype=np.float32)
    A, B = W.shape
    assert A % block == 0 and B % block == 0
    V = W.reshape(A // block, block, B // block, block).transpose(0, 2, 1, 3)
    codes, scales = _quant_groups(V.reshape(A // block, B // block, block * block))
    codes = codes.reshape(A // block, B // block, block, block).transpose(0, 2, 1, 3)
    return np.ascontiguousarray(codes.reshape(A, B)), scales


def dequant_tiles(codes, scales, block: int = 128):
    vals = e4m3_decode(codes)
    s = np.repeat(np.repeat(np.asarray(scales, np.float64), block, axis=0), block, axis=1)
    return vals * s


def token_block_offsets(offsets, block: int = 128):
    """First block index of every expert when each expert's rows are cut into
    `block`-row blocks (last one short): blk[e] = sum_{e'<e} ceil(m_e'/block)."""
    offsets = np.asarray(offsets, dtype=np.int64)
    m = np.diff(offsets)
    nb = (m + block - 1) // block
    blk = np.zeros(len(offsets), dtype=np.int64)
    blk[1:] = np.cumsum(nb)
    return blk


def quant_token_blocks(X, offsets, block: int = 128):
    """Per-column blocks of `block` consecutive rows inside each expert segment.

    codes [P][C]; scales fp32 [NB][C] where row-block b of expert e is global
    block token_block_offsets(offsets)[e] + b.
    """
    X = np.asarray(X, dtype=np.float32)
    P, C = X.shape
    blk = token_block_offsets(offsets, block)
    codes = np.zeros((P, C), dtype=np.uint8)
    scales = np.ones((int(blk[-1]), C), dtype=np.float32)
    for e in range(len(offsets) - 1):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        for b, s in enumerate(range(r0, r1, block)):
            t = min(s + block, r1)
            c_t, s_t = _quant_groups(X[s:t].T)          # one block per column
            codes[s:t] = c_t.T
            scales[blk[e] + b] = s_t
    return codes, scales


def dequant_token_blocks(codes, scales, offsets, block: int = 128):
    vals = e4m3_decode(codes)
    out = np.zeros_like(vals)
    blk = token_block_offsets(offsets, block)
    for e in range(len(offsets) - 1):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        for b, s in enumerate(range(r0, r1, block)):
            t = min(s + block, r1)
            out[s:t] = vals[s:t] * np.asarray(scales[blk[e] + b], np.float64)[None, :]
    return out
