"""Q4_0 block quantization (oracle; test infrastructure only).

The Minueza-32M -> KMCU v1 page (pnsm.cn/news/1981961.html):

* section 2: weights are cut into flat 32-element blocks of 18 bytes: bytes
  [0,2) the fp16 scale d = max|w| / 8, bytes [2,18) sixteen bytes of 4-bit
  codes, q = round(w/d) clipped to [-8, 7], stored as nibble = q + 8, low
  nibble = even index; dequant (nibble - 8) * d; 4.5 bits per weight.
* section 3: every row is zero-padded to a multiple of 32 before
  quantizing, so a block never straddles two rows; block id = r*nblk + b
  with nblk = ceil(cols/32).

Readings of the page's garbled numpy: d is 1.0 for an
all-zero block (``amax > 0`` in the comparison that lost its operator);
codes are computed with the fp32 d, the block stores fp16(d) (half-even) and
decodes with it; rint is half-to-even; the division is fp32, correctly
rounded.  A block's maximum element maps to +8 and is clipped to 7.
"""
from __future__ import annotations

import numpy as np

BLOCK = 32
BLOCK_BYTES = 18


def padded_cols(cols: int) -> int:
    return (cols + BLOCK - 1) // BLOCK * BLOCK


def blocks_per_row(cols: int) -> int:
    return padded_cols(cols) // BLOCK


def encode(w: np.ndarray) -> np.ndarray:
    """fp32 W[rows, cols] -> uint8 [rows, nblk, 18] blocks.

    Block b of a row covers columns 32b .. 32b+31; columns at or past ``cols``
    are the zero padding of section 3.  Per block (section 2): the scale is
    d = max|w| / 8 (1 for an all-zero block), stored as fp16 in bytes 0-1
    (little-endian); element j gets q = round(w_j / d) clipped to [-8, 7] and
    its nibble q + 8 goes to byte 2 + j // 2, in the low half for even j and
    the high half for odd j."""
    w = np.asarray(w, dtype=np.float32)
    rows, cols = w.shape
    nblk = blocks_per_row(cols)
    out = np.zeros((rows, nblk, BLOCK_BYTES), dtype=np.uint8)
    for b in range(nblk):
        c0 = b * BLOCK
        vals = np.zeros((rows, BLOCK), dtype=np.float32)          # the block's 32 weights, every row
        width = min(BLOCK, cols - c0)
        vals[:, :width] = w[:, c0:c0 + width]
        amax = np.max(np.abs(vals), axis=1)
        d = np.ones(rows, dtype=np.float32)
        nz = amax > 0
        d[nz] = amax[nz] / np.float32(8.0)                        # fp32, correctly rounded
        bits = d.astype("<f2").view("<u2")
        out[:, b, 0] = bits & 0xFF
        out[:, b, 1] = bits >> 8
        for j in range(BLOCK):
            q = np.clip(np.rint(vals[:, j] / d), -8, 7).astype(np.int64)   # fp32 quotient, ties to even
            out[:, b, 2 + j // 2] |= ((q + 8) << (4 * (j % 2))).astype(np.uint8)
    return out


def decode(blocks: np.ndarray, cols: int) -> np.ndarray:
    """uint8 [rows, nblk, 18] -> fp64 W_hat[rows, cols] (padding dropped)."""
    blocks = np.asarray(blocks, dtype=np.uint8)
    rows, nblk, _ = blocks.shape
    d = blocks[..., 0:2].copy().view(np.float16)[..., 0].astype(np.float64)
    packed = blocks[..., 2:]
    nib = np.empty((rows, nblk, BLOCK), dtype=np.int64)
    nib[..., 0::2] = packed & 0x0F
    nib[..., 1::2] = packed >> 4
    w = (nib - 8) * d[..., None]
    return w.reshape(rows, nblk * BLOCK)[:, :cols]


def nbytes(rows: int, cols: int) -> int:
    return rows * blocks_per_row(cols) * BLOCK_BYTES
