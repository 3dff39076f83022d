"""Weight-only low-bit quantized matmul on MI355X (gfx950).

The product is ``libbqm.so`` (HIP kernels behind the C ABI in
``include/bqm.h``); ``binding`` is its thin Python face.  The binding is
loaded on first use of one of its names, so ``inputs`` (seeded synthetic
workloads) can be imported without the library.
"""
from __future__ import annotations

__all__ = [
    "cq_pack_info", "cq_analytic_levels", "act_fwht_quant_a8", "cq_gemv", "cq_gemv_f32", "cq_gemm",
    "q4_0_gemv", "cq_pack", "q4_0_pack", "cq_codebook_fit", "CqLayout", "BqmError",
]


def __getattr__(name):
    if name in __all__:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
