"""KMCU v1 container writer: the conversion side of the loader in the C ABI.

The Minueza-32M -> KMCU v1 page (pnsm.cn/news/1981961.html), section 4 (the
header and directory tables, 64-byte aligned data) and section 5 (the
converter writes the header, then the directory, then the data).  The
payloads are given: Q4_0 blocks as q4_0_pack writes them (18 bytes per 32
columns, rows padded to whole blocks), f32 tensors as little-endian floats.

Layout choices where the page leaves freedom: the directory follows the
header (dir_offset = 128), the data starts at the first 64-byte boundary after
the directory, and every gap is zero bytes.
"""
from __future__ import annotations

import struct

F32, Q4 = 1, 2
_HEADER = 128
_RECORD = 48
# u32 fields from byte 4, in the page's order; then two f32 and total_params
_U32_FIELDS = ("version", "n_layers", "dim", "n_heads", "n_kv_heads", "head_dim", "ffn_dim",
               "vocab_size", "max_seq", "bos_id", "eos_id", "tied_embed", "n_tensors",
               "dir_offset", "data_offset")


def _up64(n: int) -> int:
    return -(-n // 64) * 64


def payload_bytes(dtype: int, rows: int, cols: int) -> int:
    if dtype == F32:
        return 4 * rows * cols
    if dtype == Q4:
        return 18 * rows * (-(-cols // 32))
    raise ValueError(f"unknown dtype {dtype}")


def write(model: dict, tensors) -> bytearray:
    """model: n_layers, dim, n_heads, n_kv_heads, head_dim, ffn_dim,
    vocab_size, max_seq, bos_id, eos_id, tied_embed, rope_theta, norm_eps.
    tensors: (name, dtype, n_rows, n_cols, payload bytes) in file order."""
    dir_offset = _HEADER
    data_offset = _up64(dir_offset + _RECORD * len(tensors))
    offsets, pos = [], data_offset
    for name, dtype, rows, cols, payload in tensors:
        if len(payload) != payload_bytes(dtype, rows, cols):
            raise ValueError(f"{name}: {len(payload)} bytes for a {rows}x{cols} tensor of dtype {dtype}")
        if len(name.encode()) > 24:
            raise ValueError(f"{name}: names hold at most 24 bytes")
        pos = _up64(pos)
        offsets.append(pos)
        pos += len(payload)
    if pos >= 1 << 32:
        raise ValueError("offsets are u32: the file must stay under 4 GiB")
    out = bytearray(pos)
    vals = dict(model, version=1, n_tensors=len(tensors), dir_offset=dir_offset, data_offset=data_offset)
    out[0:4] = b"KMCU"
    struct.pack_into("<15I", out, 4, *(int(vals[f]) for f in _U32_FIELDS))
    struct.pack_into("<ffI", out, 64, float(model["rope_theta"]), float(model["norm_eps"]),
                     sum(r * c for _, _, r, c, _ in tensors))
    for i, ((name, dtype, rows, cols, payload), off) in enumerate(zip(tensors, offsets)):
        rec = dir_offset + _RECORD * i
        raw = name.encode()
        out[rec:rec + len(raw)] = raw
        out[rec + 24] = dtype
        struct.pack_into("<4I", out, rec + 28, rows, cols, off, len(payload))
        out[off:off + len(payload)] = bytes(payload)
    return out
