"""KMCU v1 container: the oracle writer/reader pinned to the page's tables and
printed file sizes, and the C-ABI reader (kmcu_header / kmcu_tensor /
kmcu_find) checked field by field against the oracle, with its error cases.

The Minueza-32M -> KMCU v1 page (pnsm.cn/news/1981961.html), sections 1 and 4.
The C-ABI reader parses host bytes only, so these tests run without a GPU;
the upload into device memory is covered by a GPU test at the end.
"""
from __future__ import annotations

import struct

import numpy as np
import pytest

from oracle import kmcu as ok
from oracle import q4_0 as oq4
from tests.conftest import read_golden_rows

EINVAL, EALIGN, ENOTSUP = -1, -2, -3           # include/bqm.h status codes


def lib():
    from bit_quantized_matmul_amd import binding as B
    try:
        B.load_library()
    except OSError as e:                      # not built here
        pytest.skip(f"library not built: {e}")
    return B


def zero_weights(name, rows, cols):
    return np.zeros((rows, cols), np.float32)


def seeded_weights(seed):
    def w(name, rows, cols):
        rng = np.random.default_rng(seed + sum(map(ord, name)) + rows)
        return rng.standard_normal((rows, cols)).astype(np.float32) * 0.05
    return w


def seeded_norms(seed):
    def n(name):
        rng = np.random.default_rng(seed + 7 * sum(map(ord, name)))
        return (1.0 + 0.1 * rng.standard_normal(ok.MINUEZA_CONFIG["dim"])).astype(np.float32)
    return n


def image(layers=2, untied=False, seed=5):
    tensors = ok.minueza_tensors(seeded_weights(seed), seeded_norms(seed), layers,
                                 untied_head=True if untied else None)
    cfg = dict(ok.MINUEZA_CONFIG, n_layers=layers, tied_embed=0 if untied else 1)
    return ok.write(cfg, tensors), tensors


@pytest.fixture(scope="module")
def small():
    return image()


# ------------------------------------------------------------ oracle pins

def test_oracle_header_and_record_offsets_follow_the_page_table():
    rows = read_golden_rows("kmcu_layout.txt")
    hdr = {r[1]: (int(r[2]), r[3]) for r in rows if r[0] == "header"}
    rec = {r[1]: (int(r[2]), r[3]) for r in rows if r[0] == "record"}
    # distinct sentinel values in every header field, then read them back at
    # the page's offsets
    cfg = {name: 1000 + 17 * i for i, (name, _, _) in enumerate(ok.HEADER_FIELDS)}
    cfg.update(rope_theta=12345.5, norm_eps=0.25)
    tensors = [("abc", ok.F32, 1, 3, np.arange(3, dtype="<f4").tobytes()),
               ("L0.q", ok.Q4, 2, 40, oq4.encode(np.ones((2, 40), np.float32)).tobytes())]
    buf = ok.write(cfg, tensors)
    assert buf[:4] == b"KMCU" and hdr["magic"] == (0, "char4")
    fixed = dict(version=1, n_tensors=2, dir_offset=128, data_offset=ok.align(128 + 2 * 48),
                 total_params=3 + 80)
    for name, (off, typ) in hdr.items():
        if name == "magic":
            continue
        code = {"u32": "<I", "f32": "<f"}[typ]
        want = fixed.get(name, cfg[name])
        assert struct.unpack_from(code, buf, off)[0] == pytest.approx(want), name
    assert {f for f, _, _ in ok.HEADER_FIELDS} == set(hdr) - {"magic"}
    assert max(off for off, _ in hdr.values()) + 4 <= ok.HEADER_BYTES == 128
    # records: the second one, at dir_offset + 48
    r1 = 128 + 48
    assert buf[r1 + rec["name"][0]:r1 + 24] == b"L0.q" + bytes(20)
    assert buf[r1 + rec["dtype"][0]] == 2
    n_rows, n_cols, off, nb = (struct.unpack_from("<I", buf, r1 + rec[f][0])[0]
                               for f in ("n_rows", "n_cols", "offset", "nbytes"))
    assert (n_rows, n_cols) == (2, 40)
    assert nb == 2 * 2 * 18                      # 40 columns -> two 18-byte blocks per row
    assert off % 64 == 0 and buf[off:off + nb] == tensors[1][4]
    codes = {r[1]: int(r[2]) for r in rows if r[0] == "dtype"}
    assert (codes["f32"], codes["q4"]) == (ok.F32, ok.Q4)


def test_oracle_names_follow_the_page_order():
    order = [r for r in read_golden_rows("kmcu_layout.txt") if r[0] == "names"][0][1:]
    names = [t[0] for t in ok.minueza_tensors(zero_weights, lambda n: np.zeros(312, np.float32), 2)]
    per_layer = [s.replace("{i}", "0") for s in order[1:-1]]
    want = [order[0]] + per_layer + [s.replace("0", "1", 1) for s in per_layer] + [order[-1]]
    assert names == want


@pytest.mark.parametrize("untied", [False, True])
def test_oracle_full_minueza_image_has_the_printed_size(untied):
    """Section 1: 22.81 M params in 12.58 MB tied, 32.79 M in 18.07 MB untied
    (MB read as MiB), for the 10-layer model of section 1's table."""
    g = {r[0].split(":")[0]: float(r[0].split(":")[1]) for r in read_golden_rows("minueza_sizes.txt")}
    tensors = ok.minueza_tensors(zero_weights, lambda n: np.zeros(312, np.float32), 10,
                                 untied_head=True if untied else None)
    buf = ok.write(dict(ok.MINUEZA_CONFIG, tied_embed=0 if untied else 1), tensors)
    key = "untied" if untied else "tied"
    assert round(len(buf) / 2 ** 20, 2) == g[f"{key}_mib"]
    hdr, recs = ok.read(buf)
    assert round(hdr["total_params"] / 1e6, 2) == g[f"{key}_params_millions"]
    assert hdr["n_tensors"] == len(recs) == 1 + 10 * 9 + 1 + untied


def test_oracle_read_inverts_write(small):
    buf, tensors = small
    hdr, recs = ok.read(buf)
    assert [r["name"] for r in recs] == [t[0] for t in tensors]
    for r, (name, dtype, rows, cols, data) in zip(recs, tensors):
        assert (r["dtype"], r["n_rows"], r["n_cols"]) == (dtype, rows, cols)
        assert buf[r["offset"]:r["offset"] + r["nbytes"]] == data
    # a Q4_0 payload decodes to the oracle's dequantised matrix
    q = next(r for r in recs if r["name"] == "L1.down")
    blk = np.frombuffer(buf, np.uint8, q["nbytes"], q["offset"]).reshape(q["n_rows"], -1, 18)
    w = seeded_weights(5)("L1.down", 312, 1092)
    assert np.array_equal(oq4.decode(blk, 1092), oq4.decode(oq4.encode(w), 1092))


# --------------------------------------------------- C-ABI reader vs oracle

def test_abi_header_matches_oracle(small):
    B = lib()
    buf, _ = small
    hdr, _ = ok.read(buf)
    got = B.kmcu_header(buf).as_dict()
    for k, v in hdr.items():
        assert got[k] == pytest.approx(v), k


def test_abi_every_record_matches_oracle(small):
    B = lib()
    buf, _ = small
    _, recs = ok.read(buf)
    for i, r in enumerate(recs):
        assert B.kmcu_tensor(buf, i).as_dict() == r
        assert B.kmcu_find(buf, r["name"]).as_dict() == r


def test_abi_reads_the_full_minueza_directory():
    B = lib()
    tensors = ok.minueza_tensors(zero_weights, lambda n: np.zeros(312, np.float32), 10)
    buf = ok.write(ok.MINUEZA_CONFIG, tensors)
    _, recs = ok.read(buf)
    assert B.kmcu_header(buf).n_tensors == 92
    assert [B.kmcu_tensor(buf, i).as_dict() for i in range(92)] == recs
    t = B.kmcu_find(buf, "tok_embed")
    assert (t.dtype, t.n_rows, t.n_cols, t.nbytes) == (ok.Q4, 32002, 312, 32002 * 10 * 18)


def _patched(buf, off, fmt, value):
    b = bytearray(buf)
    struct.pack_into(fmt, b, off, value)
    return bytes(b)


def _status(fn):
    from bit_quantized_matmul_amd import binding as B
    try:
        fn()
    except B.BqmError as e:
        return e.code
    return 0


def test_abi_header_errors(small):
    B = lib()
    buf, _ = small
    assert _status(lambda: B.kmcu_header(b"KMC")) == EINVAL                 # truncated
    assert _status(lambda: B.kmcu_header(buf[:127])) == EINVAL
    assert _status(lambda: B.kmcu_header(b"KMCV" + buf[4:])) == EINVAL      # magic
    assert _status(lambda: B.kmcu_header(_patched(buf, 4, "<I", 2))) == ENOTSUP  # version
    assert _status(lambda: B.kmcu_header(_patched(buf, 56, "<I", 64))) == EINVAL  # dir inside header
    # directory running past the end of the file
    assert _status(lambda: B.kmcu_header(_patched(buf, 52, "<I", 10 ** 6))) == EINVAL
    assert _status(lambda: B.kmcu_header(_patched(buf, 60, "<I", len(buf) + 1))) == EINVAL


def test_abi_record_errors(small):
    B = lib()
    buf, _ = small
    hdr, recs = ok.read(buf)
    n = hdr["n_tensors"]
    assert _status(lambda: B.kmcu_tensor(buf, n)) == EINVAL
    assert _status(lambda: B.kmcu_tensor(buf, -1)) == EINVAL
    rec = 128 + 48 * 1                                            # L0.in_ln (f32)
    assert recs[1]["name"] == "L0.in_ln"
    bad = {
        "dtype": _patched(buf, rec + 24, "<B", 3),
        "zero rows": _patched(buf, rec + 28, "<I", 0),
        "nbytes": _patched(buf, rec + 40, "<I", recs[1]["nbytes"] + 4),
        "misaligned": _patched(buf, rec + 36, "<I", recs[1]["offset"] + 4),
        "before data": _patched(buf, rec + 36, "<I", 0),
        "past end": _patched(buf, rec + 36, "<I", ok.align(len(buf))),
    }
    for what, b in bad.items():
        assert _status(lambda: B.kmcu_tensor(b, 1)) == EINVAL, what
        assert _status(lambda: B.kmcu_find(b, "L0.in_ln")) == EINVAL, what
    # a Q4_0 record's nbytes counts padded blocks: 1092 columns -> 35 blocks
    d = next(r for r in recs if r["name"] == "L0.down")
    assert d["nbytes"] == 312 * 35 * 18
    assert _status(lambda: B.kmcu_find(buf, "L9.q")) == EINVAL              # no such name
    assert _status(lambda: B.kmcu_find(buf, "L0")) == EINVAL                # prefix only


def test_abi_upload_rejects_bad_arguments_before_any_copy(small):
    """Argument checks return before the device is touched (no GPU needed)."""
    import ctypes
    B = lib()
    buf, _ = small
    t = B.kmcu_find(buf, "L0.q")
    L = B.load_library()
    arr = np.frombuffer(buf, np.uint8)
    p, n = ctypes.c_void_p(arr.ctypes.data), arr.nbytes
    assert L.kmcu_upload(p, n, ctypes.byref(t), None, None) == EINVAL
    assert L.kmcu_upload(p, n, None, ctypes.c_void_p(4096), None) == EINVAL
    assert L.kmcu_upload(p, n, ctypes.byref(t), ctypes.c_void_p(4096 + 8), None) == EALIGN
    for field, value in (("dtype", 3), ("n_rows", 0)):
        bad = B.KmcuTensor.from_buffer_copy(t)
        setattr(bad, field, value)
        assert L.kmcu_upload(p, n, ctypes.byref(bad), ctypes.c_void_p(4096), None) == EINVAL, field
    short = B.KmcuTensor.from_buffer_copy(t)
    short.nbytes -= 18
    assert L.kmcu_upload(p, n, ctypes.byref(short), ctypes.c_void_p(4096), None) == EINVAL
    assert L.kmcu_upload(p, t.offset + t.nbytes - 1, ctypes.byref(t), ctypes.c_void_p(4096), None) == EINVAL


def test_package_writer_matches_oracle_byte_for_byte(small):
    """The package's writer (the conversion side) lays a file out exactly as
    the oracle does, for the same payloads."""
    from bit_quantized_matmul_amd import kmcu as pk
    buf, tensors = small
    cfg = dict(ok.MINUEZA_CONFIG, n_layers=2)
    assert bytes(pk.write(cfg, tensors)) == buf
    odd = [("a", ok.F32, 1, 1, b"\0\0\x80\x3f"), ("b" * 24, ok.Q4, 3, 33, bytes(range(108)))]
    assert bytes(pk.write(cfg, odd)) == ok.write(cfg, odd)
    with pytest.raises(ValueError):
        pk.write(cfg, [("c", ok.Q4, 1, 33, bytes(18))])          # 33 columns take two blocks
    with pytest.raises(ValueError):
        pk.write(cfg, [("d" * 25, ok.F32, 1, 1, bytes(4))])


def test_abi_upload_data_checks_before_copying(small):
    """kmcu_upload_data validates the header, every record and dst before the
    copy (these cases return without touching the device)."""
    import ctypes
    B = lib()
    L = B.load_library()
    buf, _ = small
    hdr, recs = ok.read(buf)

    def call(b, dst, nbytes):
        arr = np.frombuffer(b, np.uint8)
        return L.kmcu_upload_data(ctypes.c_void_p(arr.ctypes.data), arr.nbytes, dst, nbytes, None)

    need = len(buf) - hdr["data_offset"]
    assert call(buf, None, need) == EINVAL
    assert call(buf, ctypes.c_void_p(4096), need - 1) == EINVAL
    assert call(buf, ctypes.c_void_p(4096 + 4), need) == EALIGN
    bad = _patched(buf, 128 + 48 * 7 + 24, "<B", 0)              # one bad record, anywhere
    assert call(bad, ctypes.c_void_p(4096), need) == EINVAL
    assert call(_patched(buf, 60, "<I", hdr["data_offset"] + 8), ctypes.c_void_p(4096), need) == EINVAL


# ------------------------------------------------------ GPU: upload + GEMV

@pytest.mark.gpu
def test_upload_then_q4_0_gemv_matches_oracle(small):
    """Every Q4_0 matrix of a 2-layer Minueza-shaped file, uploaded with
    kmcu_upload, lands byte for byte and feeds q4_0_gemv to the oracle's
    product; the f32 norms land as floats."""
    import torch
    from bit_quantized_matmul_amd import binding as B
    from bit_quantized_matmul_amd import inputs
    from oracle import matmul as omm
    buf, _ = small
    _, recs = ok.read(buf)
    rng = np.random.default_rng(808)
    for r in recs:
        t = B.kmcu_find(buf, r["name"])
        d = B.kmcu_upload(buf, t)
        raw = np.frombuffer(buf, np.uint8, r["nbytes"], r["offset"])
        assert np.array_equal(d.cpu().numpy(), raw), r["name"]
        if r["dtype"] == ok.F32:
            assert np.array_equal(d.view(torch.float32).cpu().numpy(), raw.view("<f4")), r["name"]
            continue
        rows, cols = r["n_rows"], r["n_cols"]
        x = inputs.activations(rng, 1, cols)
        y = B.q4_0_gemv(d, rows, cols, torch.from_numpy(x).cuda())
        torch.cuda.synchronize()
        ref = omm.q4_0_reference(raw.reshape(rows, -1, 18), cols, x)
        assert omm.rel_l2(y.cpu().numpy(), ref) <= 1e-3, r["name"]


@pytest.mark.gpu
def test_load_whole_image_in_one_copy():
    """kmcu_load: one copy of the data region from pinned host memory; every
    tensor's view holds its file bytes, and the views keep 64-byte alignment."""
    import torch
    from bit_quantized_matmul_amd import binding as B
    buf, _ = image(layers=3, untied=True, seed=9)
    pinned = torch.empty((len(buf),), dtype=torch.uint8, pin_memory=True)
    pinned.numpy()[:] = np.frombuffer(buf, np.uint8)
    for src in (buf, pinned):
        h, tensors = B.kmcu_load(src)
        _, recs = ok.read(buf)
        assert h.n_tensors == len(tensors) == len(recs)
        for r in recs:
            t, view = tensors[r["name"]]
            assert t.as_dict() == r
            assert view.data_ptr() % 64 == 0
            raw = np.frombuffer(buf, np.uint8, r["nbytes"], r["offset"])
            assert np.array_equal(view.cpu().numpy(), raw), r["name"]


def test_abi_edge_cases_empty_file_and_full_length_name():
    """A file with no tensors parses (and its empty data region uploads as a
    no-op before any device call); a name of exactly 24 bytes has no NUL in
    the record and still comes back whole."""
    import ctypes
    B = lib()
    L = B.load_library()
    empty = ok.write(ok.MINUEZA_CONFIG, [])
    h = B.kmcu_header(empty)
    assert (h.n_tensors, h.dir_offset, h.data_offset) == (0, 128, 128) and len(empty) == 128
    assert _status(lambda: B.kmcu_tensor(empty, 0)) == EINVAL
    assert _status(lambda: B.kmcu_find(empty, "tok_embed")) == EINVAL
    arr = np.frombuffer(empty, np.uint8)
    assert L.kmcu_upload_data(ctypes.c_void_p(arr.ctypes.data), arr.nbytes, ctypes.c_void_p(4096), 0, None) == 0
    name = "x" * 24
    buf = ok.write(ok.MINUEZA_CONFIG, [(name, ok.F32, 2, 3, np.arange(6, dtype="<f4").tobytes())])
    t = B.kmcu_find(buf, name)
    assert t.name.decode() == name and (t.n_rows, t.n_cols, t.nbytes) == (2, 3, 24)
    assert _status(lambda: B.kmcu_find(buf, name + "y")) == EINVAL       # 25 bytes never match
    from bit_quantized_matmul_amd import kmcu as pk
    assert bytes(pk.write(ok.MINUEZA_CONFIG, [(name, ok.F32, 2, 3, np.arange(6, dtype="<f4").tobytes())])) == buf
