"""KMCU v1 container writer and reader (oracle; test infrastructure only).

The Minueza-32M -> KMCU v1 page (pnsm.cn/news/1981961.html), section 4:

* a 128-byte little-endian header: magic "KMCU", then u32 version (1),
  n_layers, dim, n_heads, n_kv_heads, head_dim, ffn_dim, vocab_size, max_seq,
  bos_id, eos_id, tied_embed (1: the output head reuses tok_embed), n_tensors,
  dir_offset, data_offset, then f32 rope_theta and norm_eps, then u32
  total_params; the rest of the 128 bytes is zero;
* at dir_offset, n_tensors 48-byte records: name (24 bytes, zero-padded),
  u8 dtype (1 = f32, 2 = Q4_0) at byte 24, then u32 n_rows (28), n_cols (32:
  the columns before padding to 32), offset (36: absolute file offset) and
  nbytes (40);
* tensor data from data_offset, every tensor starting 64-byte aligned;
* names tok_embed, L{i}.in_ln, L{i}.q, L{i}.k, L{i}.v, L{i}.o, L{i}.post_ln,
  L{i}.gate, L{i}.up, L{i}.down, final_norm (section 4's naming list, in
  that order); norms are f32, matrices Q4_0 (section 1: --force-tie keeps
  no separate output head).

Readings where the page leaves freedom: the directory follows the header directly
(dir_offset = 128) and the data the directory (data_offset = the first
64-byte boundary after it); unused header and record bytes are zero.
"""
from __future__ import annotations

import struct

from . import q4_0

HEADER_BYTES = 128
RECORD_BYTES = 48
ALIGN = 64
MAGIC = b"KMCU"
F32, Q4 = 1, 2
# (field, byte offset, struct code) in the page's header table order
HEADER_FIELDS = (
    ("version", 4, "I"), ("n_layers", 8, "I"), ("dim", 12, "I"), ("n_heads", 16, "I"),
    ("n_kv_heads", 20, "I"), ("head_dim", 24, "I"), ("ffn_dim", 28, "I"), ("vocab_size", 32, "I"),
    ("max_seq", 36, "I"), ("bos_id", 40, "I"), ("eos_id", 44, "I"), ("tied_embed", 48, "I"),
    ("n_tensors", 52, "I"), ("dir_offset", 56, "I"), ("data_offset", 60, "I"),
    ("rope_theta", 64, "f"), ("norm_eps", 68, "f"), ("total_params", 72, "I"),
)


def align(n: int, a: int = ALIGN) -> int:
    return (n + a - 1) // a * a


def tensor_bytes(dtype: int, rows: int, cols: int) -> int:
    return q4_0.nbytes(rows, cols) if dtype == Q4 else 4 * rows * cols


def write(config: dict, tensors) -> bytes:
    """config: the header's model fields; tensors: (name, dtype, rows, cols, data bytes)
    in file order.  Returns the file's bytes."""
    n = len(tensors)
    dir_offset = HEADER_BYTES
    data_offset = align(dir_offset + RECORD_BYTES * n)
    hdr = dict(config)
    hdr.update(version=1, n_tensors=n, dir_offset=dir_offset, data_offset=data_offset,
               total_params=sum(r * c for _, _, r, c, _ in tensors))
    out = bytearray(HEADER_BYTES)
    out[0:4] = MAGIC
    for name, off, code in HEADER_FIELDS:
        struct.pack_into("<" + code, out, off, hdr[name])
    out += bytes(data_offset - HEADER_BYTES)
    pos = data_offset
    placed = []
    for name, dtype, rows, cols, data in tensors:
        assert len(data) == tensor_bytes(dtype, rows, cols), name
        pos = align(pos)
        placed.append((name, dtype, rows, cols, pos, len(data)))
        pos += len(data)
    for i, (name, dtype, rows, cols, off, nb) in enumerate(placed):
        rec = dir_offset + RECORD_BYTES * i
        raw = name.encode()
        assert len(raw) <= 24, name
        out[rec:rec + len(raw)] = raw
        out[rec + 24] = dtype
        struct.pack_into("<IIII", out, rec + 28, rows, cols, off, nb)
    for (name, dtype, rows, cols, data), (_, _, _, _, off, nb) in zip(tensors, placed):
        if len(out) < off:
            out += bytes(off - len(out))
        out += data
    return bytes(out)


def read(buf: bytes):
    """File bytes -> (header dict, [record dict ...]); asserts the page's layout."""
    assert buf[0:4] == MAGIC
    hdr = {name: struct.unpack_from("<" + code, buf, off)[0] for name, off, code in HEADER_FIELDS}
    assert hdr["version"] == 1
    recs = []
    for i in range(hdr["n_tensors"]):
        rec = hdr["dir_offset"] + RECORD_BYTES * i
        name = bytes(buf[rec:rec + 24]).split(b"\0", 1)[0].decode()
        dtype = buf[rec + 24]
        rows, cols, off, nb = struct.unpack_from("<IIII", buf, rec + 28)
        assert off % ALIGN == 0 and off + nb <= len(buf)
        assert nb == tensor_bytes(dtype, rows, cols)
        recs.append(dict(name=name, dtype=dtype, n_rows=rows, n_cols=cols, offset=off, nbytes=nb))
    return hdr, recs


MINUEZA_CONFIG = dict(n_layers=10, dim=312, n_heads=12, n_kv_heads=4, head_dim=26, ffn_dim=1092,
                      vocab_size=32002, max_seq=2048, bos_id=1, eos_id=32000, tied_embed=1,
                      rope_theta=10000.0, norm_eps=1e-6)


def minueza_tensors(weights, norm_of, layers: int, untied_head=None):
    """The page's tensor list for a Minueza-shaped model: weights(label, rows,
    cols) -> fp32 matrix, norm_of(name) -> fp32 vector of dim."""
    cfg = MINUEZA_CONFIG
    dim, ffn, vocab = cfg["dim"], cfg["ffn_dim"], cfg["vocab_size"]
    kv = cfg["n_kv_heads"] * cfg["head_dim"]

    def q4(name, rows, cols):
        return (name, Q4, rows, cols, q4_0.encode(weights(name, rows, cols)).tobytes())

    def f32(name):
        v = norm_of(name)
        return (name, F32, 1, dim, v.astype("<f4").tobytes())

    out = [q4("tok_embed", vocab, dim)]
    for i in range(layers):
        out.append(f32(f"L{i}.in_ln"))
        out += [q4(f"L{i}.q", dim, dim), q4(f"L{i}.k", kv, dim), q4(f"L{i}.v", kv, dim),
                q4(f"L{i}.o", dim, dim)]
        out.append(f32(f"L{i}.post_ln"))
        out += [q4(f"L{i}.gate", ffn, dim), q4(f"L{i}.up", ffn, dim), q4(f"L{i}.down", dim, ffn)]
    out.append(f32("final_norm"))
    if untied_head is not None:
        out.append(q4("lm_head", vocab, dim))
    return out
