"""Host-side checks of the C ABI (CPU only: no call here reaches a device)."""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np
import pytest

from oracle import codebook as ocb
from oracle import cq as ocq
from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "bqm.h")


def declared_functions() -> list[str]:
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", src, flags=re.M)


@pytest.fixture(scope="module")
def lib():
    from bit_quantized_matmul_amd import binding
    if not os.path.exists(binding.library_path()):
        pytest.fail("libbqm.so is not built (run python -m bit_quantized_matmul_amd.build)")
    return binding.load_library()


def test_header_declares_the_abi():
    names = declared_functions()
    for required in ("cq_pack_info", "act_fwht_quant_a8", "cq_gemv", "cq_gemv_f32", "cq_gemm", "q4_0_gemv",
                     "q4_0_gemm", "cq_pack", "q4_0_pack", "cq_codebook_fit", "cq_analytic_levels",
                     "bqm_strerror"):
        assert required in names


def test_library_exports_every_declared_symbol(lib):
    from bit_quantized_matmul_amd import binding
    names = declared_functions()
    for n in names:
        assert hasattr(lib, n), f"libbqm.so does not export {n}"
    assert set(names) == set(binding.EXPORTED)


@pytest.mark.parametrize("rows,cols,code", [(512, 512, 4), (14336, 4096, 4), (104, 1024, 3), (7, 256, 1),
                                            (5, 384, 5), (4096, 14336, 2), (1, 128, 3), (14336, 4096, 6),
                                            (3, 640, 6), (1, 128, 6)])
def test_pack_info_matches_oracle(lib, rows, cols, code):
    from bit_quantized_matmul_amd import binding
    assert binding.cq_pack_info(rows, cols, 128, code).as_dict() == ocq.pack_info(rows, cols, 128, code)


def test_pack_info_rejects_bad_arguments(lib):
    from bit_quantized_matmul_amd import binding
    lay = binding.CqLayout()
    for args in [(4, 100, 128, 4), (4, 128, 128, 7), (0, 128, 128, 4), (4, 128, 96, 4), (4, 128, 128, 0),
                 (4, 100, 128, 6)]:
        assert lib.cq_pack_info(*args, ctypes.byref(lay)) == binding.BQM_EINVAL
    assert lib.cq_pack_info(4, 128, 128, 4, None) == binding.BQM_EINVAL


def test_analytic_levels_match_oracle(lib):
    from bit_quantized_matmul_amd import binding
    assert np.array_equal(binding.cq_analytic_levels(1), ocb.analytic_levels(1))
    assert np.array_equal(binding.cq_analytic_levels(5), ocb.analytic_levels(5))
    assert np.array_equal(binding.cq_analytic_levels(6), ocb.analytic_levels(5))   # base-3: the ternary set
    out = (ctypes.c_float * 3)()
    assert lib.cq_analytic_levels(4, out) == binding.BQM_EINVAL


def test_device_entry_points_validate_before_touching_a_device(lib):
    """Invalid calls return an error code; none of them reaches HIP (no GPU here)."""
    from bit_quantized_matmul_amd import binding
    lay = binding.cq_pack_info(256, 512, 128, 4)
    bad = binding.cq_pack_info(256, 512, 128, 4)
    bad.idx_bytes += 1                                  # inconsistent layout
    cb = (ctypes.c_float * 16)(*([0.5] * 16))
    p = ctypes.c_void_p(4096)                           # never dereferenced: checks fail first
    E = binding
    assert lib.act_fwht_quant_a8(None, 1, 128, 128, p, p, None) == E.BQM_EINVAL
    assert lib.act_fwht_quant_a8(p, 1, 100, 128, p, p, None) == E.BQM_EINVAL
    assert lib.act_fwht_quant_a8(p, 1, 256, 64, p, p, None) == E.BQM_ENOTSUP
    assert lib.cq_gemv(p, ctypes.byref(bad), cb, p, p, 1, p, None) == E.BQM_EINVAL
    assert lib.cq_gemv(p, ctypes.byref(lay), None, p, p, 1, p, None) == E.BQM_EINVAL   # codebook needed
    assert lib.cq_gemv(p, ctypes.byref(lay), cb, p, p, 0, p, None) == E.BQM_EINVAL
    assert lib.cq_gemv(p, ctypes.byref(lay), cb, p, p, 33, p, None) == E.BQM_ENOTSUP
    nonbf16 = (ctypes.c_float * 16)(*([0.1] * 16))     # 0.1 is not bfloat16-representable
    assert lib.cq_gemv(p, ctypes.byref(lay), nonbf16, p, p, 1, p, None) == E.BQM_EINVAL
    tern = binding.cq_pack_info(256, 512, 128, 5)
    assert lib.cq_gemv(p, ctypes.byref(tern), cb, p, p, 1, p, None) == E.BQM_EINVAL     # analytic: NULL
    g64 = binding.cq_pack_info(256, 512, 64, 4)
    assert lib.cq_gemm(p, ctypes.byref(g64), cb, p, p, 4, p, None) == E.BQM_ENOTSUP
    assert lib.cq_gemv(ctypes.c_void_p(4097), ctypes.byref(lay), cb, p, p, 1, p, None) == E.BQM_EALIGN
    big = binding.cq_pack_info(8, 32768, 128, 4)
    assert lib.cq_gemv_f32(p, ctypes.byref(big), cb, p, 1, p, None, None, None) == E.BQM_ENOTSUP
    over = binding.cq_pack_info(8, 16512, 128, 4)                      # one group past the fused limit
    assert lib.cq_gemv_f32(p, ctypes.byref(over), cb, p, 1, p, None, None, None) == E.BQM_ENOTSUP
    # ... which runs in two launches into code buffers, 16-byte aligned, up to cq_gemv's width
    assert lib.cq_gemv_f32(p, ctypes.byref(over), cb, p, 1, p, ctypes.c_void_p(4100), p, None) == E.BQM_EALIGN
    assert lib.cq_gemv_f32(p, ctypes.byref(over), cb, p, 17, p, p, p, None) == E.BQM_ENOTSUP
    wide = binding.cq_pack_info(8, 36992, 128, 4)                      # one group past the int8 limit
    assert lib.cq_gemv(p, ctypes.byref(wide), cb, p, p, 1, p, None) == E.BQM_ENOTSUP
    assert lib.cq_gemv_f32(p, ctypes.byref(wide), cb, p, 1, p, p, p, None) == E.BQM_ENOTSUP
    assert lib.cq_gemv_f32(p, ctypes.byref(lay), cb, None, 1, p, None, None, None) == E.BQM_EINVAL
    assert lib.cq_gemv_f32(p, ctypes.byref(lay), cb, p, 1, p, ctypes.c_void_p(4098), None, None) == E.BQM_EALIGN
    # base-3 ternary: the GEMV up to 16 tokens and 128 groups a row (the GEMM
    # takes any column count, within the 32-bit offsets), the fused path
    # needs the code buffers
    t3 = binding.cq_pack_info(256, 512, 128, 6)
    assert lib.cq_gemv(p, ctypes.byref(t3), cb, p, p, 1, p, None) == E.BQM_EINVAL      # analytic: NULL
    assert lib.cq_gemv(p, ctypes.byref(t3), None, p, p, 17, p, None) == E.BQM_ENOTSUP
    t3wide = binding.cq_pack_info(8, 16512, 128, 6)                                   # 129 groups
    assert lib.cq_gemv(p, ctypes.byref(t3wide), None, p, p, 2, p, None) == E.BQM_ENOTSUP
    assert lib.cq_gemm(p, ctypes.byref(t3wide), None, p, p, 1 << 16, p, None) == E.BQM_ENOTSUP   # m * cols >= 2^30
    assert lib.cq_gemm(p, ctypes.byref(t3), cb, p, p, 4, p, None) == E.BQM_EINVAL      # analytic: NULL
    assert lib.cq_gemv_f32(p, ctypes.byref(t3), None, p, 1, p, None, None, None) == E.BQM_ENOTSUP
    assert lib.cq_gemv_f32(p, ctypes.byref(t3), None, p, 1, p, ctypes.c_void_p(4100), p, None) == E.BQM_EALIGN
    t3big = binding.cq_pack_info(8, 16512, 128, 6)                                      # 129 groups
    assert lib.cq_gemv(p, ctypes.byref(t3big), None, p, p, 1, p, None) == E.BQM_ENOTSUP
    assert lib.q4_0_gemv(None, 4, 312, p, 1, p, None) == E.BQM_EINVAL
    assert lib.q4_0_gemv(p, 4, 312, p, 17, p, None) == E.BQM_ENOTSUP
    assert lib.q4_0_gemm(p, 4, 312, p, 0, p, None) == E.BQM_EINVAL
    assert lib.q4_0_gemm(p, 4, 312, None, 8, p, None) == E.BQM_EINVAL
    assert lib.q4_0_gemm(p, 4, 312, ctypes.c_void_p(4100), 8, p, None) == E.BQM_EALIGN
    assert lib.q4_0_gemm(p, 4, 1 << 20, p, 1024, p, None) == E.BQM_ENOTSUP     # m * cols * 4 >= 2^31
    # q4_0_gemv addresses its blocks with 32-bit offsets: 2^27 rows of one block is past 2^31 bytes
    assert lib.q4_0_gemv(p, 1 << 27, 32, p, 1, p, None) == E.BQM_ENOTSUP
    assert lib.q4_0_gemv(p, (1 << 27) - 1, 1, ctypes.c_void_p(4100), 1, p, None) == E.BQM_ENOTSUP
    # A8 without the rotation: group 1 takes any k; other groups are not built
    assert lib.act_fwht_quant_a8(p, 1, 312, 2, p, p, None) == E.BQM_ENOTSUP
    assert lib.act_fwht_quant_a8(p, 1, 312, 3, p, p, None) == E.BQM_EINVAL
    assert lib.act_fwht_quant_a8(p, 1, 65537, 1, p, p, None) == E.BQM_ENOTSUP
    assert lib.act_fwht_quant_a8(ctypes.c_void_p(4100), 1, 312, 1, p, p, None) == E.BQM_EALIGN
    for fn in (lib.q4_0_gemv_a8, lib.q4_0_gemm_a8):
        assert fn(None, 4, 312, p, p, 1, p, None) == E.BQM_EINVAL
        assert fn(p, 4, 312, p, p, 0, p, None) == E.BQM_EINVAL
        assert fn(p, 4, 312, ctypes.c_void_p(4100), p, 1, p, None) == E.BQM_EALIGN
        assert fn(p, 1 << 27, 32, p, p, 1, p, None) == E.BQM_ENOTSUP          # blocks past 2^31 bytes
    assert lib.q4_0_gemv_a8(p, 4, 312, p, p, 17, p, None) == E.BQM_ENOTSUP
    assert lib.q4_0_gemm_a8(p, 4, 1 << 20, p, p, 4096, p, None) == E.BQM_ENOTSUP   # codes past 2^31 bytes
    # the fused A8 Q4_0 GEMV: fp32 activations, codes of one token within a workgroup's LDS
    f = lib.q4_0_gemv_a8_f32
    assert f(None, 4, 312, p, 1, p, None, None, None) == E.BQM_EINVAL
    assert f(p, 4, 312, p, 0, p, None, None, None) == E.BQM_EINVAL
    assert f(p, 4, 0, p, 1, p, None, None, None) == E.BQM_EINVAL
    assert f(p, 4, 312, p, 17, p, None, None, None) == E.BQM_ENOTSUP
    assert f(p, 4, 54593, p, 1, p, None, None, None) == E.BQM_ENOTSUP            # 1707 blocks a row
    assert f(p, 1 << 27, 32, p, 1, p, None, None, None) == E.BQM_ENOTSUP         # blocks past 2^31 bytes
    assert f(ctypes.c_void_p(4100), 4, 312, p, 1, p, None, None, None) == E.BQM_EALIGN
    assert f(p, 4, 312, ctypes.c_void_p(4098), 1, p, None, None, None) == E.BQM_EALIGN
    assert f(p, 4, 312, p, 1, p, None, ctypes.c_void_p(4098), None) == E.BQM_EALIGN
    # the lookup-table GEMV: binary and ternary only, widths its LDS tables hold
    assert lib.cq_gemv_lut(p, ctypes.byref(lay), p, p, 1, p, None) == E.BQM_ENOTSUP       # 4-bit
    b1 = binding.cq_pack_info(64, 8192, 128, 1)
    assert lib.cq_gemv_lut(p, ctypes.byref(b1), p, p, 0, p, None) == E.BQM_EINVAL
    assert lib.cq_gemv_lut(p, ctypes.byref(b1), p, p, 17, p, None) == E.BQM_ENOTSUP
    assert lib.cq_gemv_lut(p, ctypes.byref(binding.cq_pack_info(64, 8320, 128, 1)), p, p, 1, p, None) == E.BQM_ENOTSUP
    assert lib.cq_gemv_lut(p, ctypes.byref(binding.cq_pack_info(64, 8320, 128, 5)), p, p, 1, p, None) == E.BQM_ENOTSUP
    assert lib.cq_gemv_lut(ctypes.c_void_p(4100), ctypes.byref(b1), p, p, 1, p, None) == E.BQM_EALIGN
    assert lib.cq_pack(p, ctypes.byref(bad), cb, p, None, None) == E.BQM_EINVAL
    assert lib.q4_0_pack(p, 0, 312, p, None) == E.BQM_EINVAL
    assert lib.cq_codebook_fit(p, 1 << 20, 16, 200, None, p, None) == E.BQM_ENOTSUP
    assert lib.cq_codebook_fit(p, 1000, 6, 200, None, p, None) == E.BQM_EINVAL
    assert binding.strerror(E.BQM_EALIGN) == "misaligned pointer"


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    from bit_quantized_matmul_amd import binding
    monkeypatch.setattr(binding, "_LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(binding, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        binding.load_library()


def test_binding_checks_shapes_before_any_call(lib):
    """Every wrapper compares each tensor with the layout / row and column
    arguments and raises ValueError before a pointer reaches the library (CPU
    tensors here: a call that passed the shape checks would stop at the device
    check, whose message differs)."""
    import torch

    from bit_quantized_matmul_amd import binding as B
    lay = B.cq_pack_info(64, 256, 128, 4)
    cb = np.linspace(-1, 1, 16).astype(np.float32)
    blob = torch.zeros(lay.total_bytes, dtype=torch.uint8)
    q = torch.zeros((2, 256), dtype=torch.int8)
    sc = torch.ones(2)
    cases = [
        (lambda: B.cq_gemv(blob, lay, cb, torch.zeros((2, 128), dtype=torch.int8), sc), "q must have shape"),
        (lambda: B.cq_gemv(blob, lay, cb, q, torch.ones(3)), "scale must have shape"),
        (lambda: B.cq_gemv(blob, lay, cb, q, sc, y=torch.zeros(2, 63)), "y must have shape"),
        (lambda: B.cq_gemv(blob[:-64], lay, cb, q, sc), "blob must hold"),
        (lambda: B.cq_gemv(blob, lay, cb[:8], q, sc), "codebook must hold"),
        (lambda: B.cq_gemv(blob, lay, cb, q, sc), "CUDA/HIP tensor"),            # shapes right
        (lambda: B.cq_gemm(blob, lay, cb, torch.zeros((5, 255), dtype=torch.int8), torch.ones(5)), "q must"),
        (lambda: B.cq_gemm(blob, lay, cb, q, torch.ones(1)), "scale must have shape"),
        (lambda: B.cq_gemv_f32(blob, lay, cb, torch.zeros(2, 512)), "x must have shape"),
        (lambda: B.cq_gemv_f32(blob, lay, cb, torch.zeros(2, 256), q_out=torch.zeros((2, 255), dtype=torch.int8),
                               scale_out=sc), "q_out must have shape"),
        (lambda: B.cq_gemv_f32(blob, lay, cb, torch.zeros(2, 256), scale_out=torch.ones(4)), "scale_out must"),
        (lambda: B.act_fwht_quant_a8(torch.zeros(2, 256), q=torch.zeros((2, 128), dtype=torch.int8)), "q must"),
        (lambda: B.act_fwht_quant_a8(torch.zeros(256)), "x must be 2-D"),
        (lambda: B.cq_pack(torch.zeros(64, 128), lay, cb), "w must have shape"),
        (lambda: B.cq_pack(torch.zeros(64, 256), lay, cb, blob=blob[:100]), "blob must hold"),
        (lambda: B.q4_0_gemv(torch.zeros(100, dtype=torch.uint8), 4, 312, torch.zeros(1, 312)), "blocks must hold"),
        (lambda: B.q4_0_gemv(torch.zeros(4 * 10 * 18, dtype=torch.uint8), 4, 312, torch.zeros(1, 300)), "x must"),
        (lambda: B.q4_0_gemv(torch.zeros(4 * 10 * 18, dtype=torch.uint8), 4, 312, torch.zeros(1, 312),
                             y=torch.zeros(1, 5)), "y must have shape"),
        (lambda: B.q4_0_gemm(torch.zeros(4 * 10 * 18, dtype=torch.uint8), 4, 312, torch.zeros(7, 311)), "x must"),
        (lambda: B.q4_0_pack(torch.zeros(4, 312), blocks=torch.zeros(10, dtype=torch.uint8)), "blocks must"),
        (lambda: B.cq_codebook_fit(torch.zeros(1000, dtype=torch.float64), 16, table=torch.zeros(8)), "table must"),
    ]
    for fn, msg in cases:
        with pytest.raises(ValueError, match=msg):
            fn()
