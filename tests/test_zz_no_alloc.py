"""cq_gemv_f32_noalloc (the entry point that allocates nothing) against
cq_gemv_f32 with caller-given code buffers: the same route and kernels, so y
must match bit for bit, and both stay within the element-wise bound of the
oracle.  Two calls in a row share the device scratch, the second with a
smaller input."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from bit_quantized_matmul_amd import binding as B
from bit_quantized_matmul_amd import inputs
from oracle import a8 as oa8
from oracle import cq as ocq
from tests import parity as P

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _case(rng, rows, cols, code, batch, codebooks):
    w = inputs.weight_matrix(rng, rows, cols, outliers=True)
    x = inputs.activations(rng, batch, cols)
    lv = ocq.levels_for(code, codebooks)
    idx, n16 = ocq.encode(w, 128, code, lv)
    cb = None if code in (ocq.BINARY, ocq.TERNARY, ocq.TERNARY_B3) else codebooks[code]
    return x, lv, idx, n16, ocq.make_blob(idx, n16, 128, code), cb


def _with_buffers(blob, lay, cb, x):
    batch = x.shape[0]
    q_out = torch.empty((batch, lay.cols), dtype=torch.int8, device=DEV)
    s_out = torch.empty((batch,), dtype=torch.float32, device=DEV)
    return B.cq_gemv_f32(blob, lay, cb, x, q_out=q_out, scale_out=s_out)


# (code, rows, cols, batch) pairs: the first call large (the scratch's full
# 16 x 16384 codes on the matrix cores, or base-3 at its widest), the second
# smaller on another route
@pytest.mark.parametrize("first,second", [
    ((4, 300, 16384, 16), (4, 200, 1024, 3)),
    ((1, 129, 4096, 8), (2, 70, 512, 1)),
    ((6, 100, 8192, 16), (6, 33, 512, 2)),
    ((3, 64, 16384, 1), (5, 50, 4096, 4)),
])
def test_noalloc_matches_cq_gemv_f32(first, second, codebooks):
    rng = np.random.default_rng(1700 + first[2] + second[2])
    for code, rows, cols, batch in (first, second):
        x, lv, idx, n16, blob_h, cb = _case(rng, rows, cols, code, batch, codebooks)
        lay = B.cq_pack_info(rows, cols, 128, code)
        blob = torch.from_numpy(blob_h).to(DEV)
        dx = torch.from_numpy(x).to(DEV)
        y = torch.full((batch, rows), np.nan, dtype=torch.float32, device=DEV)
        B.cq_gemv_f32_noalloc(blob, lay, cb, dx, y)
        ref = _with_buffers(blob, lay, cb, dx)
        torch.cuda.synchronize()
        got, want = y.cpu().numpy(), ref.cpu().numpy()
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (code, rows, cols, batch)
        q, s = oa8.act_quant_a8(x, 128, "fp32")
        tol = P.TOL_F32 if code == ocq.TERNARY_B3 else P.cq_gemv_tol(cols, batch)
        P.check_cq(got, idx, n16, 128, code, lv, q, s, tol, f"noalloc code {code} {rows}x{cols} b{batch}")


def test_noalloc_rejects_sizes_past_the_scratch(codebooks):
    lib = B.load_library()
    import ctypes
    p = ctypes.c_void_p(4096)
    cb = (ctypes.c_float * 16)(*codebooks[4])
    big = B.cq_pack_info(8, 16512, 128, 4)
    assert lib.cq_gemv_f32_noalloc(p, ctypes.byref(big), cb, p, 1, p, None) == B.BQM_ENOTSUP
    lay = B.cq_pack_info(8, 1024, 128, 4)
    assert lib.cq_gemv_f32_noalloc(p, ctypes.byref(lay), cb, p, 17, p, None) == B.BQM_ENOTSUP
