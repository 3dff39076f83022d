"""CQ (Cactus Quant) encode, pack and decode (oracle; test infrastructure only).

What the pages fix (Needle .cact/W4A8 article, section 1 and section 3; the
mmap article's passage on the CQ format):

* Matmul weights are pre-transposed to [out, in]; quant groups run along the
  reduction axis (in), 128 wide by default.
* Each group is rotated by the normalized Walsh-Hadamard transform H, its
  direction is matched to the nearest entry of a shared Lloyd-Max codebook
  (only the indices are stored), and its L2 norm is stored as FP16.
* Reconstruction: w_group = (codebook[idx] * norm) H.
* Indices are packed LSB-first: each 8 indices are OR'd into a 64-bit word,
  the low nibble holding the even column.
* Bits codes: 2/3/4 use the fitted codebooks cb2/cb3/cb4; 5 is ternary and 1
  binary, both with analytic levels.
* Ternary weights also come packed as base-3 digits, five per byte (1.6 bits
  per weight), where 2-bit fields spend 2 bits (the llama.cpp TV-box / iPad
  page weighs the two against each other in its speed-up table, the 2-bit
  ternary layout of its section 18: 2-bit fields decode in fewer CPU
  operations, base-3 digits take less memory).

Readings taken where the pages are silent or garbled:

* Scale: the levels are on the N(0,1) scale, so the stored norm is the true
  L2 norm of the (normalized-H) rotated group and the quantized direction is
  t = sqrt(G) * y / ||y||; decode is w = norm/sqrt(G) * H cb[idx], which is
  norm/G * H_u cb[idx].
* Nearest level per coordinate, ties to the lower index.  A zero group has
  t = 0 and so gets the level nearest 0 (lower on a tie).
* Packing is a dense LSB-first b-bit stream per row (8 indices fill exactly
  b bytes).  Ternary uses 2-bit fields holding 0/1/2; field value 3 is never
  written and decodes to 0.
* Precision of the encode: fp64 throughout, in this operation order:
  u = H_u w (butterfly, fp64); ss = sum of u_i*u_i, i ascending, each
  product rounded then added; r = sqrt(ss); norm = r / sqrt(G), rounded
  once to fp16 (half-even); t_i = u_i * (sqrt(G) / r) when r > 0, else 0.
  (u/r equals y/||y|| exactly in real arithmetic.)
* Layout of a packed blob: the index rows back to back, then the fp16 norms
  [rows][cols/G] starting at the next 64-byte boundary, total rounded up to 64.
* Base-3 ternary (code 6, same levels and encode as code 5): each group is
  ceil(G/5) bytes (26 for G = 128); byte j holds the group's indices 5j ..
  5j+4 as sum_i idx[5j+i] * 3**i (the first index least significant, as in
  the LSB-first packing); positions past the group end hold digit 1, the zero
  level.  A row is its groups' bytes back to back.
"""
from __future__ import annotations

import numpy as np

from . import codebook as _cb
from .fp import fp16_rne
from .hadamard import fwht_u

BINARY, B2, B3, B4, TERNARY, TERNARY_B3 = 1, 2, 3, 4, 5, 6
# 0: not fixed-width fields (base-3 digits, five per byte)
INDEX_BITS = {BINARY: 1, B2: 2, B3: 3, B4: 4, TERNARY: 2, TERNARY_B3: 0}
NUM_LEVELS = {BINARY: 2, B2: 4, B3: 8, B4: 16, TERNARY: 3, TERNARY_B3: 3}
TRITS_PER_BYTE = 5
TRIT_PAD = 1          # digit of the positions past a group's end: the zero level
BLOB_ALIGN = 64


def pack_info(rows: int, cols: int, group: int, code: int) -> dict:
    """Byte layout of a packed CQ matrix (mirrors the C ABI's cq_layout)."""
    if code not in INDEX_BITS:
        raise ValueError(f"unknown bits code {code}")
    if rows < 1 or cols < 1 or group < 2 or group & (group - 1):
        raise ValueError("bad shape or group")
    if cols % group:
        raise ValueError("cols must be a multiple of group")
    ib = INDEX_BITS[code]
    if code == TERNARY_B3:
        idx_row_bytes = (cols // group) * trit_bytes(group)
    else:
        if (cols * ib) % 8:
            raise ValueError("row does not fill whole bytes")
        idx_row_bytes = cols * ib // 8
    idx_bytes = rows * idx_row_bytes
    norms_offset = _round_up(idx_bytes, BLOB_ALIGN)
    norms_count = rows * (cols // group)
    total = _round_up(norms_offset + 2 * norms_count, BLOB_ALIGN)
    return dict(rows=rows, cols=cols, group=group, bits=code, index_bits=ib,
                levels=NUM_LEVELS[code], idx_row_bytes=idx_row_bytes,
                idx_bytes=idx_bytes, norms_offset=norms_offset,
                norms_count=norms_count, total_bytes=total)


def _round_up(x: int, a: int) -> int:
    return (x + a - 1) // a * a


def trit_bytes(group: int) -> int:
    """Bytes of one base-3 packed group: five digits a byte."""
    return -(-group // TRITS_PER_BYTE)


def levels_for(code: int, codebooks: dict | None = None) -> np.ndarray:
    """fp32 level table for a bits code (ascending)."""
    if code in (BINARY, TERNARY):
        return _cb.analytic_levels(code)
    if code == TERNARY_B3:                        # the ternary set, packed base-3
        return _cb.analytic_levels(TERNARY)
    if codebooks is None or code not in codebooks:
        raise ValueError(f"bits code {code} needs its fitted codebook")
    lv = np.asarray(codebooks[code], dtype=np.float32)
    if lv.shape != (NUM_LEVELS[code],):
        raise ValueError("codebook has the wrong number of levels")
    return lv


def nearest_level(t: np.ndarray, levels: np.ndarray) -> np.ndarray:
    """Index of the nearest level per element; lower index on an exact tie."""
    lv = np.asarray(levels, dtype=np.float32).astype(np.float64)
    best = np.zeros(t.shape, dtype=np.int64)
    best_d = np.abs(t - lv[0])
    for l in range(1, len(lv)):
        d = np.abs(t - lv[l])
        better = d < best_d                      # strict: ties keep the lower l
        best = np.where(better, l, best)
        best_d = np.where(better, d, best_d)
    return best


def encode(w: np.ndarray, group: int, code: int, levels: np.ndarray):
    """Encode fp32 W[rows, cols] -> (idx uint8 [rows, cols], norm16 fp16 [rows, cols/G]).

    Raises ``OverflowError`` when a group norm does not fit fp16 and
    ``ValueError`` on non-finite weights.
    """
    w = np.asarray(w, dtype=np.float32)
    if not np.all(np.isfinite(w)):
        raise ValueError("non-finite weight")
    rows, cols = w.shape
    pack_info(rows, cols, group, code)
    ng = cols // group
    u = fwht_u(w.astype(np.float64).reshape(rows, ng, group))
    ss = np.zeros((rows, ng), dtype=np.float64)
    for i in range(group):                        # fixed order: i ascending
        ss = ss + u[..., i] * u[..., i]
    r = np.sqrt(ss)
    sqrt_g = np.sqrt(np.float64(group))
    norm = r / sqrt_g
    with np.errstate(divide="ignore", invalid="ignore"):
        scale = np.where(r > 0, sqrt_g / np.where(r > 0, r, 1.0), 0.0)
    t = u * scale[..., None]
    idx = nearest_level(t, levels).astype(np.uint8).reshape(rows, cols)
    n16 = np.array([fp16_rne(v) for v in norm.ravel()], dtype=np.float64)
    if not np.all(np.isfinite(n16)):
        raise OverflowError("group norm overflows fp16")
    return idx, n16.astype(np.float16).reshape(rows, ng)


def pack_indices(idx: np.ndarray, index_bits: int) -> np.ndarray:
    """LSB-first dense bit stream per row: index j occupies bits [b*j, b*j+b).

    Built 8 indices at a time: OR ``idx[8u+s] << (b*s)`` into one 64-bit word
    and emit its low b bytes little-endian.  For b = 4 the low nibble of each
    byte is the even column.
    """
    idx = np.asarray(idx, dtype=np.uint64)
    rows, cols = idx.shape
    b = index_bits
    if cols % 8:
        raise ValueError("pack works on whole units of 8 indices")
    if np.any(idx >> np.uint64(b)):
        raise ValueError("index does not fit the field width")
    units = idx.reshape(rows, cols // 8, 8)
    word = np.zeros((rows, cols // 8), dtype=np.uint64)
    for s in range(8):
        word |= units[..., s] << np.uint64(b * s)
    out = np.zeros((rows, cols // 8, b), dtype=np.uint8)
    for k in range(b):
        out[..., k] = ((word >> np.uint64(8 * k)) & np.uint64(0xFF)).astype(np.uint8)
    return out.reshape(rows, cols * b // 8)


def unpack_indices(packed: np.ndarray, cols: int, index_bits: int) -> np.ndarray:
    """Inverse of ``pack_indices``."""
    packed = np.asarray(packed, dtype=np.uint8)
    rows = packed.shape[0]
    b = index_bits
    units = packed.reshape(rows, cols // 8, b).astype(np.uint64)
    word = np.zeros((rows, cols // 8), dtype=np.uint64)
    for k in range(b):
        word |= units[..., k] << np.uint64(8 * k)
    mask = np.uint64((1 << b) - 1)
    idx = np.zeros((rows, cols // 8, 8), dtype=np.uint8)
    for s in range(8):
        idx[..., s] = ((word >> np.uint64(b * s)) & mask).astype(np.uint8)
    return idx.reshape(rows, cols)


def pack_trits(idx: np.ndarray, group: int) -> np.ndarray:
    """Base-3 packing per group: byte j = sum_i idx[5j+i] * 3**i over the
    group's positions 5j .. 5j+4, positions past the group holding TRIT_PAD."""
    idx = np.asarray(idx, dtype=np.int64)
    rows, cols = idx.shape
    if np.any((idx < 0) | (idx > 2)):
        raise ValueError("base-3 packing holds indices 0, 1, 2 only")
    ng, nb = cols // group, trit_bytes(group)
    digits = np.full((rows, ng, nb * TRITS_PER_BYTE), TRIT_PAD, dtype=np.int64)
    digits[:, :, :group] = idx.reshape(rows, ng, group)
    digits = digits.reshape(rows, ng, nb, TRITS_PER_BYTE)
    value = np.zeros((rows, ng, nb), dtype=np.int64)
    for i in range(TRITS_PER_BYTE):
        value += digits[..., i] * 3 ** i
    return value.astype(np.uint8).reshape(rows, ng * nb)


def unpack_trits(packed: np.ndarray, cols: int, group: int) -> np.ndarray:
    """Inverse of ``pack_trits`` (bytes above 242 are not base-3 digits)."""
    packed = np.asarray(packed, dtype=np.int64)
    rows = packed.shape[0]
    if np.any(packed > 3 ** TRITS_PER_BYTE - 1):
        raise ValueError("byte value above 242")
    ng, nb = cols // group, trit_bytes(group)
    v = packed.reshape(rows, ng, nb)
    digits = np.zeros((rows, ng, nb, TRITS_PER_BYTE), dtype=np.uint8)
    for i in range(TRITS_PER_BYTE):
        digits[..., i] = v % 3
        v = v // 3
    return digits.reshape(rows, ng, nb * TRITS_PER_BYTE)[:, :, :group].reshape(rows, cols)


def make_blob(idx: np.ndarray, norm16: np.ndarray, group: int, code: int) -> np.ndarray:
    """Assemble the packed blob bytes (indices, 64-aligned fp16 norms)."""
    rows, cols = idx.shape
    info = pack_info(rows, cols, group, code)
    blob = np.zeros(info["total_bytes"], dtype=np.uint8)
    packed = pack_trits(idx, group) if code == TERNARY_B3 else pack_indices(idx, info["index_bits"])
    blob[: info["idx_bytes"]] = packed.ravel()
    nb = np.ascontiguousarray(norm16, dtype=np.float16).view(np.uint8).ravel()
    blob[info["norms_offset"]: info["norms_offset"] + nb.size] = nb
    return blob


def split_blob(blob: np.ndarray, rows: int, cols: int, group: int, code: int):
    """Blob bytes -> (idx uint8 [rows, cols], norm16 fp16 [rows, cols/G])."""
    info = pack_info(rows, cols, group, code)
    blob = np.asarray(blob, dtype=np.uint8)
    packed = blob[: info["idx_bytes"]].reshape(rows, info["idx_row_bytes"])
    idx = (unpack_trits(packed, cols, group) if code == TERNARY_B3
           else unpack_indices(packed, cols, info["index_bits"]))
    nb = blob[info["norms_offset"]: info["norms_offset"] + 2 * info["norms_count"]]
    return idx, nb.view(np.float16).reshape(rows, cols // group).copy()


def level_values(idx: np.ndarray, code: int, levels: np.ndarray) -> np.ndarray:
    """cb[idx] in fp64; a ternary field value 3 decodes to 0."""
    lv = np.asarray(levels, dtype=np.float32).astype(np.float64)
    ext = np.concatenate([lv, np.zeros(max(1 << INDEX_BITS[code], len(lv)) - len(lv))])
    return ext[np.asarray(idx, dtype=np.int64)]


def decode(idx: np.ndarray, norm16: np.ndarray, group: int, code: int, levels: np.ndarray) -> np.ndarray:
    """Reconstruct W_hat [rows, cols] in fp64: w_g = norm/G * H_u cb[idx_g]."""
    rows, cols = idx.shape
    ng = cols // group
    c = level_values(idx, code, levels).reshape(rows, ng, group)
    n = np.asarray(norm16, dtype=np.float16).astype(np.float64).reshape(rows, ng, 1)
    return (fwht_u(c) * (n / group)).reshape(rows, cols)


def quantization_mse(w: np.ndarray, w_hat: np.ndarray) -> float:
    """Relative squared error ||w - w_hat||^2 / ||w||^2."""
    w = np.asarray(w, dtype=np.float64)
    return float(np.sum((w - w_hat) ** 2) / np.sum(w * w))


__all__ = [
    "BINARY", "B2", "B3", "B4", "TERNARY", "INDEX_BITS", "NUM_LEVELS",
    "pack_info", "levels_for", "nearest_level", "encode", "pack_indices",
    "unpack_indices", "make_blob", "split_blob", "level_values", "decode",
    "quantization_mse",
]
