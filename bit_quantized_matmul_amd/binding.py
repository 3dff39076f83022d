"""Thin Python binding of libbqm's C ABI (include/bqm.h).

Argument marshalling only: every computation runs in the HIP kernels of
``libbqm.so``.  PyTorch supplies device memory and the current HIP stream.
There is no fallback: if the library is missing or the call fails, an
exception is raised.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbqm.so")

BQM_OK, BQM_EINVAL, BQM_EALIGN, BQM_ENOTSUP, BQM_EDEVICE, BQM_ERANGE = 0, -1, -2, -3, -4, -5
BINARY, B2, B3, B4, TERNARY, TERNARY_B3 = 1, 2, 3, 4, 5, 6
STATUS_NONFINITE, STATUS_NORM_OVERFLOW = 1, 2
GROUP = 128

EXPORTED = (
    "cq_pack_info", "cq_analytic_levels", "act_fwht_quant_a8", "cq_gemv", "cq_gemv_f32",
    "cq_gemm", "q4_0_gemv", "q4_0_gemm", "cq_pack", "q4_0_pack", "cq_codebook_fit", "bqm_strerror",
    "kmcu_header", "kmcu_tensor", "kmcu_find", "kmcu_upload", "kmcu_upload_data", "cq_gemv_f32_noalloc",
    "q4_0_gemv_a8", "q4_0_gemm_a8", "cq_gemv_lut", "q4_0_gemv_a8_f32",
)
KMCU_F32, KMCU_Q4 = 1, 2


class BqmError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} failed: {code} ({strerror(code)})")
        self.code = code


class CqLayout(ctypes.Structure):
    _fields_ = [
        ("rows", ctypes.c_int32), ("cols", ctypes.c_int32), ("group", ctypes.c_int32),
        ("bits", ctypes.c_int32), ("index_bits", ctypes.c_int32), ("levels", ctypes.c_int32),
        ("idx_row_bytes", ctypes.c_int64), ("idx_bytes", ctypes.c_int64),
        ("norms_offset", ctypes.c_int64), ("norms_count", ctypes.c_int64),
        ("total_bytes", ctypes.c_int64),
    ]

    def as_dict(self) -> dict:
        return {name: int(getattr(self, name)) for name, _ in self._fields_}


class KmcuHeader(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint32) for n in (
        "version", "n_layers", "dim", "n_heads", "n_kv_heads", "head_dim", "ffn_dim", "vocab_size",
        "max_seq", "bos_id", "eos_id", "tied_embed", "n_tensors", "dir_offset", "data_offset")] + [
        ("rope_theta", ctypes.c_float), ("norm_eps", ctypes.c_float), ("total_params", ctypes.c_uint32)]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


class KmcuTensor(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 25), ("dtype", ctypes.c_uint32), ("n_rows", ctypes.c_uint32),
                ("n_cols", ctypes.c_uint32), ("offset", ctypes.c_uint32), ("nbytes", ctypes.c_uint32)]

    def as_dict(self) -> dict:
        d = {name: getattr(self, name) for name, _ in self._fields_}
        d["name"] = self.name.decode()
        return d


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load_library() -> ctypes.CDLL:
    """Load libbqm.so, raising if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                           "`python -m bit_quantized_matmul_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I, I64, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.POINTER(ctypes.c_float)
    LP = ctypes.POINTER(CqLayout)
    sig = {
        "cq_pack_info": ([I, I, I, I, LP], I),
        "cq_analytic_levels": ([I, F], I),
        "act_fwht_quant_a8": ([P, I, I, I, P, P, P], I),
        "cq_gemv": ([P, LP, F, P, P, I, P, P], I),
        "cq_gemv_f32": ([P, LP, F, P, I, P, P, P, P], I),
        "cq_gemv_f32_noalloc": ([P, LP, F, P, I, P, P], I),
        "cq_gemv_lut": ([P, LP, P, P, I, P, P], I),
        "cq_gemm": ([P, LP, F, P, P, I, P, P], I),
        "q4_0_gemv": ([P, I, I, P, I, P, P], I),
        "q4_0_gemm": ([P, I, I, P, I, P, P], I),
        "q4_0_gemv_a8": ([P, I, I, P, P, I, P, P], I),
        "q4_0_gemm_a8": ([P, I, I, P, P, I, P, P], I),
        "q4_0_gemv_a8_f32": ([P, I, I, P, I, P, P, P, P], I),
        "cq_pack": ([P, LP, F, P, P, P], I),
        "q4_0_pack": ([P, I, I, P, P], I),
        "cq_codebook_fit": ([P, I64, I, I, P, P, P], I),
        "bqm_strerror": ([I], ctypes.c_char_p),
        "kmcu_header": ([P, ctypes.c_uint64, ctypes.POINTER(KmcuHeader)], I),
        "kmcu_tensor": ([P, ctypes.c_uint64, I, ctypes.POINTER(KmcuTensor)], I),
        "kmcu_find": ([P, ctypes.c_uint64, ctypes.c_char_p, ctypes.POINTER(KmcuTensor)], I),
        "kmcu_upload": ([P, ctypes.c_uint64, ctypes.POINTER(KmcuTensor), P, P], I),
        "kmcu_upload_data": ([P, ctypes.c_uint64, P, ctypes.c_uint64, P], I),
    }
    for name, (args, ret) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ret
    _lib = lib
    return lib


def strerror(code: int) -> str:
    return load_library().bqm_strerror(code).decode()


def _check(fn: str, code: int) -> None:
    if code != BQM_OK:
        raise BqmError(fn, code)


# ------------------------------------------------------------------ host calls

def cq_pack_info(rows: int, cols: int, group: int, bits: int) -> CqLayout:
    lay = CqLayout()
    _check("cq_pack_info", load_library().cq_pack_info(rows, cols, group, bits, ctypes.byref(lay)))
    return lay


def cq_analytic_levels(bits: int) -> np.ndarray:
    n = 2 if bits == BINARY else 3
    out = (ctypes.c_float * 3)()
    _check("cq_analytic_levels", load_library().cq_analytic_levels(bits, out))
    return np.array(out[:n], dtype=np.float32)


def _codebook_ptr(codebook, levels=None):
    """Host fp32 array (or None) -> (ctypes pointer, keep-alive object).  The
    library reads `levels` values from it, so a shorter array is rejected."""
    if codebook is None:
        return None, None
    arr = np.ascontiguousarray(np.asarray(codebook.cpu() if hasattr(codebook, "cpu") else codebook,
                                          dtype=np.float32)).ravel()
    if levels is not None and arr.size != levels:
        raise ValueError(f"codebook must hold {levels} levels, got {arr.size}")
    return arr.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), arr


# ---------------------------------------------------------------- device calls

def _torch():
    import torch
    return torch


def _stream():
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _shape(t, shape, name):
    """Check a tensor's shape before any pointer reaches the library (a wrong
    shape would send device reads or writes past the tensor)."""
    got = tuple(getattr(t, "shape", ()))
    if got != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {got}")


def _at_least(t, nbytes, name):
    """Check that a byte buffer holds at least `nbytes` elements."""
    n = t.numel() if hasattr(t, "numel") else np.asarray(t).size
    if n < nbytes:
        raise ValueError(f"{name} must hold at least {nbytes} bytes, got {n}")


def _rows2d(t, cols, name):
    """A 2-D [batch, cols] tensor's batch."""
    if getattr(t, "ndim", 0) != 2 or t.shape[1] != cols:
        raise ValueError(f"{name} must have shape [batch, {cols}], got {tuple(getattr(t, 'shape', ()))}")
    if t.shape[0] < 1:
        raise ValueError(f"{name} must have at least one row")
    return int(t.shape[0])


def _dev(t, dtype, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA/HIP tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def act_fwht_quant_a8(x, group: int = GROUP, q=None, scale=None):
    """x fp32 [m, k] -> (q int8 [m, k], scale fp32 [m])."""
    torch = _torch()
    if getattr(x, "ndim", 0) != 2:
        raise ValueError(f"x must be 2-D [m, k], got {tuple(getattr(x, 'shape', ()))}")
    m, k = x.shape
    if q is None:
        q = torch.empty((m, k), dtype=torch.int8, device=x.device)
    if scale is None:
        scale = torch.empty((m,), dtype=torch.float32, device=x.device)
    _shape(q, (m, k), "q")
    _shape(scale, (m,), "scale")
    _check("act_fwht_quant_a8", load_library().act_fwht_quant_a8(
        _dev(x, torch.float32, "x"), m, k, group, _dev(q, torch.int8, "q"),
        _dev(scale, torch.float32, "scale"), _stream()))
    return q, scale


def cq_gemv(blob, layout: CqLayout, codebook, q, scale, y=None):
    """Packed CQ [rows, cols] x int8 q [batch, cols] -> fp32 y [batch, rows]."""
    torch = _torch()
    batch = _rows2d(q, layout.cols, "q")
    _at_least(blob, layout.total_bytes, "blob")
    _shape(scale, (batch,), "scale")
    if y is None:
        y = torch.empty((batch, layout.rows), dtype=torch.float32, device=q.device)
    _shape(y, (batch, layout.rows), "y")
    cb, _keep = _codebook_ptr(codebook, layout.levels)
    _check("cq_gemv", load_library().cq_gemv(
        _dev(blob, torch.uint8, "blob"), ctypes.byref(layout), cb, _dev(q, torch.int8, "q"),
        _dev(scale, torch.float32, "scale"), batch, _dev(y, torch.float32, "y"), _stream()))
    return y


def cq_gemv_lut(blob, layout: CqLayout, q, scale, y=None):
    """Binary / ternary CQ [rows, cols] x int8 q [batch, cols] -> fp32 y [batch, rows],
    the lookup-table kernel."""
    torch = _torch()
    batch = _rows2d(q, layout.cols, "q")
    _at_least(blob, layout.total_bytes, "blob")
    _shape(scale, (batch,), "scale")
    if y is None:
        y = torch.empty((batch, layout.rows), dtype=torch.float32, device=q.device)
    _shape(y, (batch, layout.rows), "y")
    _check("cq_gemv_lut", load_library().cq_gemv_lut(
        _dev(blob, torch.uint8, "blob"), ctypes.byref(layout), _dev(q, torch.int8, "q"),
        _dev(scale, torch.float32, "scale"), batch, _dev(y, torch.float32, "y"), _stream()))
    return y


def cq_gemv_f32(blob, layout: CqLayout, codebook, x, y=None, q_out=None, scale_out=None):
    """Packed CQ [rows, cols] x fp32 x [batch, cols] -> fp32 y [batch, rows]; the A8
    step runs inside the GEMV launch (optional q_out / scale_out receive the codes)."""
    torch = _torch()
    batch = _rows2d(x, layout.cols, "x")
    _at_least(blob, layout.total_bytes, "blob")
    if y is None:
        y = torch.empty((batch, layout.rows), dtype=torch.float32, device=x.device)
    _shape(y, (batch, layout.rows), "y")
    if q_out is not None:
        _shape(q_out, (batch, layout.cols), "q_out")
    if scale_out is not None:
        _shape(scale_out, (batch,), "scale_out")
    cb, _keep = _codebook_ptr(codebook, layout.levels)
    qo = _dev(q_out, torch.int8, "q_out") if q_out is not None else None
    so = _dev(scale_out, torch.float32, "scale_out") if scale_out is not None else None
    _check("cq_gemv_f32", load_library().cq_gemv_f32(
        _dev(blob, torch.uint8, "blob"), ctypes.byref(layout), cb, _dev(x, torch.float32, "x"),
        batch, _dev(y, torch.float32, "y"), qo, so, _stream()))
    return y


def cq_gemv_f32_noalloc(blob, layout: CqLayout, codebook, x, y):
    """cq_gemv_f32 with the codes staged in the library's device scratch: the
    call allocates nothing (y is the caller's)."""
    torch = _torch()
    batch = _rows2d(x, layout.cols, "x")
    _at_least(blob, layout.total_bytes, "blob")
    _shape(y, (batch, layout.rows), "y")
    cb, _keep = _codebook_ptr(codebook, layout.levels)
    _check("cq_gemv_f32_noalloc", load_library().cq_gemv_f32_noalloc(
        _dev(blob, torch.uint8, "blob"), ctypes.byref(layout), cb, _dev(x, torch.float32, "x"),
        batch, _dev(y, torch.float32, "y"), _stream()))
    return y


def cq_gemm(blob, layout: CqLayout, codebook, q, scale, y=None):
    """Packed CQ [rows, cols] x int8 q [m, cols] -> fp32 y [m, rows] (matrix cores)."""
    torch = _torch()
    m = _rows2d(q, layout.cols, "q")
    _at_least(blob, layout.total_bytes, "blob")
    _shape(scale, (m,), "scale")
    if y is None:
        y = torch.empty((m, layout.rows), dtype=torch.float32, device=q.device)
    _shape(y, (m, layout.rows), "y")
    cb, _keep = _codebook_ptr(codebook, layout.levels)
    _check("cq_gemm", load_library().cq_gemm(
        _dev(blob, torch.uint8, "blob"), ctypes.byref(layout), cb, _dev(q, torch.int8, "q"),
        _dev(scale, torch.float32, "scale"), m, _dev(y, torch.float32, "y"), _stream()))
    return y


def q4_0_gemv(blocks, rows: int, cols: int, x, y=None):
    """Q4_0 blocks [rows, ceil(cols/32), 18] x fp32 x [batch, cols] -> fp32 y [batch, rows]."""
    torch = _torch()
    batch = _rows2d(x, cols, "x")
    _at_least(blocks, q4_0_nbytes(rows, cols), "blocks")
    if y is None:
        y = torch.empty((batch, rows), dtype=torch.float32, device=x.device)
    _shape(y, (batch, rows), "y")
    _check("q4_0_gemv", load_library().q4_0_gemv(
        _dev(blocks, torch.uint8, "blocks"), rows, cols, _dev(x, torch.float32, "x"), batch,
        _dev(y, torch.float32, "y"), _stream()))
    return y


def q4_0_gemm(blocks, rows: int, cols: int, x, y=None):
    """Q4_0 blocks [rows, ceil(cols/32), 18] x fp32 x [m, cols] -> fp32 y [m, rows]."""
    torch = _torch()
    m = _rows2d(x, cols, "x")
    _at_least(blocks, q4_0_nbytes(rows, cols), "blocks")
    if y is None:
        y = torch.empty((m, rows), dtype=torch.float32, device=x.device)
    _shape(y, (m, rows), "y")
    _check("q4_0_gemm", load_library().q4_0_gemm(
        _dev(blocks, torch.uint8, "blocks"), rows, cols, _dev(x, torch.float32, "x"), m,
        _dev(y, torch.float32, "y"), _stream()))
    return y


def _q4_0_a8(fn, blocks, rows, cols, q, scale, y):
    torch = _torch()
    n = _rows2d(q, cols, "q")
    _at_least(blocks, q4_0_nbytes(rows, cols), "blocks")
    _shape(scale, (n,), "scale")
    if y is None:
        y = torch.empty((n, rows), dtype=torch.float32, device=q.device)
    _shape(y, (n, rows), "y")
    _check(fn, getattr(load_library(), fn)(
        _dev(blocks, torch.uint8, "blocks"), rows, cols, _dev(q, torch.int8, "q"),
        _dev(scale, torch.float32, "scale"), n, _dev(y, torch.float32, "y"), _stream()))
    return y


def q4_0_gemv_a8(blocks, rows: int, cols: int, q, scale, y=None):
    """Q4_0 blocks x int8 codes q [batch, cols] (act_fwht_quant_a8, group 1) -> fp32 y [batch, rows]."""
    return _q4_0_a8("q4_0_gemv_a8", blocks, rows, cols, q, scale, y)


def q4_0_gemm_a8(blocks, rows: int, cols: int, q, scale, y=None):
    """Q4_0 blocks x int8 codes q [m, cols] -> fp32 y [m, rows] on the int8 matrix cores."""
    return _q4_0_a8("q4_0_gemm_a8", blocks, rows, cols, q, scale, y)


def q4_0_gemv_a8_f32(blocks, rows: int, cols: int, x, y=None, q_out=None, scale_out=None):
    """Q4_0 blocks x fp32 x [batch, cols], quantized per token to int8 in the
    same launch (act_fwht_quant_a8, group 1) -> fp32 y [batch, rows];
    q_out [batch, cols] int8 and scale_out [batch] receive the codes and
    scales when given."""
    torch = _torch()
    batch = _rows2d(x, cols, "x")
    _at_least(blocks, q4_0_nbytes(rows, cols), "blocks")
    if y is None:
        y = torch.empty((batch, rows), dtype=torch.float32, device=x.device)
    _shape(y, (batch, rows), "y")
    qp = sp = None
    if q_out is not None:
        _shape(q_out, (batch, cols), "q_out")
        qp = _dev(q_out, torch.int8, "q_out")
    if scale_out is not None:
        _shape(scale_out, (batch,), "scale_out")
        sp = _dev(scale_out, torch.float32, "scale_out")
    _check("q4_0_gemv_a8_f32", load_library().q4_0_gemv_a8_f32(
        _dev(blocks, torch.uint8, "blocks"), rows, cols, _dev(x, torch.float32, "x"), batch,
        _dev(y, torch.float32, "y"), qp, sp, _stream()))
    return y


# ---------------------------------------------------------------- KMCU container

def _host_bytes(buf):
    """A host byte buffer (bytes, bytearray, numpy uint8, CPU torch uint8
    tensor, pinned or not) -> (pointer, size, keep-alive)."""
    if isinstance(buf, (bytes, bytearray, memoryview)):
        arr = np.frombuffer(buf, dtype=np.uint8)
        return ctypes.c_void_p(arr.ctypes.data), arr.nbytes, arr
    if not isinstance(buf, np.ndarray):
        torch = _torch()
        if isinstance(buf, torch.Tensor):
            if buf.is_cuda or buf.dtype != torch.uint8 or not buf.is_contiguous():
                raise ValueError("file must be a contiguous host uint8 tensor")
            return ctypes.c_void_p(buf.data_ptr()), buf.numel(), buf
    if buf.dtype != np.uint8 or not buf.flags.c_contiguous:
        raise ValueError("file must be a contiguous uint8 array")
    return ctypes.c_void_p(buf.ctypes.data), buf.nbytes, buf


def kmcu_header(file) -> KmcuHeader:
    p, n, _keep = _host_bytes(file)
    h = KmcuHeader()
    _check("kmcu_header", load_library().kmcu_header(p, n, ctypes.byref(h)))
    return h


def kmcu_tensor(file, index: int) -> KmcuTensor:
    p, n, _keep = _host_bytes(file)
    t = KmcuTensor()
    _check("kmcu_tensor", load_library().kmcu_tensor(p, n, index, ctypes.byref(t)))
    return t


def kmcu_find(file, name: str) -> KmcuTensor:
    p, n, _keep = _host_bytes(file)
    t = KmcuTensor()
    _check("kmcu_find", load_library().kmcu_find(p, n, name.encode(), ctypes.byref(t)))
    return t


def kmcu_upload(file, tensor: KmcuTensor, dst=None):
    """Copy one tensor of the file into a device buffer (uint8 [nbytes]); the
    call waits for the copy, so the file buffer may be released afterwards."""
    torch = _torch()
    if dst is None:
        dst = torch.empty((tensor.nbytes,), dtype=torch.uint8, device="cuda")
    _at_least(dst, tensor.nbytes, "dst")
    p, n, _keep = _host_bytes(file)
    _check("kmcu_upload", load_library().kmcu_upload(p, n, ctypes.byref(tensor),
                                                     _dev(dst, torch.uint8, "dst"), _stream()))
    torch.cuda.current_stream().synchronize()
    return dst


def kmcu_upload_data(file, dst=None):
    """The file's whole data region into one device buffer (uint8), one copy;
    returns it.  The call waits for the copy."""
    torch = _torch()
    p, n, _keep = _host_bytes(file)
    if dst is None:
        h = kmcu_header(file)
        dst = torch.empty((n - h.data_offset,), dtype=torch.uint8, device="cuda")
    _check("kmcu_upload_data", load_library().kmcu_upload_data(p, n, _dev(dst, torch.uint8, "dst"),
                                                               dst.numel(), _stream()))
    torch.cuda.current_stream().synchronize()
    return dst


def kmcu_load(file):
    """Parse a KMCU v1 file and move its tensors to the device in one copy.
    Returns (header, {name: (record, uint8 device view of its bytes)}); the
    views share one allocation, each at its file offset minus data_offset."""
    h = kmcu_header(file)
    data = kmcu_upload_data(file)
    out = {}
    for i in range(h.n_tensors):
        t = kmcu_tensor(file, i)
        start = t.offset - h.data_offset
        out[t.name.decode()] = (t, data[start:start + t.nbytes])
    return h, out


def cq_pack(w, layout: CqLayout, codebook, blob=None, status=None):
    """fp32 W [rows, cols] -> packed blob (uint8 [total_bytes]) on the device."""
    torch = _torch()
    _shape(w, (layout.rows, layout.cols), "w")
    if blob is None:
        blob = torch.empty((layout.total_bytes,), dtype=torch.uint8, device=w.device)
    _at_least(blob, layout.total_bytes, "blob")
    if status is not None and status.numel() < 1:
        raise ValueError("status must hold one int32")
    cb, _keep = _codebook_ptr(codebook, layout.levels)
    st = _dev(status, torch.int32, "status") if status is not None else None
    _check("cq_pack", load_library().cq_pack(
        _dev(w, torch.float32, "w"), ctypes.byref(layout), cb, _dev(blob, torch.uint8, "blob"),
        st, _stream()))
    return blob


def q4_0_nbytes(rows: int, cols: int) -> int:
    return rows * ((cols + 31) // 32) * 18


def q4_0_pack(w, blocks=None):
    """fp32 W [rows, cols] -> Q4_0 blocks (uint8 [rows*ceil(cols/32)*18])."""
    torch = _torch()
    if getattr(w, "ndim", 0) != 2:
        raise ValueError(f"w must be 2-D [rows, cols], got {tuple(getattr(w, 'shape', ()))}")
    rows, cols = w.shape
    if blocks is None:
        blocks = torch.empty((q4_0_nbytes(rows, cols),), dtype=torch.uint8, device=w.device)
    _at_least(blocks, q4_0_nbytes(rows, cols), "blocks")
    _check("q4_0_pack", load_library().q4_0_pack(
        _dev(w, torch.float32, "w"), rows, cols, _dev(blocks, torch.uint8, "blocks"), _stream()))
    return blocks


def cq_codebook_fit(samples, levels: int, iters: int = 200, table=None, raw=None):
    """Lloyd-Max fit on device fp64 samples -> (table fp32 [levels], raw fp64 [levels])."""
    torch = _torch()
    if getattr(samples, "ndim", 0) != 1:
        raise ValueError("samples must be 1-D")
    if table is None:
        table = torch.empty((levels,), dtype=torch.float32, device=samples.device)
    if raw is None:
        raw = torch.empty((levels,), dtype=torch.float64, device=samples.device)
    _shape(table, (levels,), "table")
    _shape(raw, (levels,), "raw")
    _check("cq_codebook_fit", load_library().cq_codebook_fit(
        _dev(samples, torch.float64, "samples"), samples.numel(), levels, iters,
        _dev(raw, torch.float64, "raw"), _dev(table, torch.float32, "table"), _stream()))
    return table, raw
