"""CPU oracle for the bit-quantized matmul: TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, fp64 (numpy) restatement of what the
quantized-matmul path computes.  It exists so that the HIP path can be
checked against an independent implementation.  Only the test suite, the
smoke check in ``__graft_entry__`` and the ``cpu_baseline`` leg of
``bench.py`` may import it; the product library never does, and it shares
no code, tables or constants with the HIP sources.

Sources (the pages are cited by title and section):

* "14MB holds 45M parameters: dissecting Needle's .cact file and W4A8
  quantization" (wmrh.cn/news/49311), section 1 (CQ codebook quantization)
  and section 3 (pre-transposed [out,in] layout, GEMV/GEMM).
* "Parse-free loading: mmap tensors and Needle's cold start"
  (kwkr.cn/news/556663), the passage on the CQ format and the analytic
  ternary/binary sets.
* The Minueza-32M -> KMCU v1 page (pnsm.cn/news/1981961.html), section 2
  (Q4_0 block quantization) and section 3 (row alignment to 32).

Modules:

* ``hadamard``  Sylvester Hadamard matrix and the butterfly FWHT.
* ``codebook``  Lloyd-Max fits (sampled and by quadrature), analytic sets.
* ``cq``        CQ encode / pack / decode and the blob layout.
* ``a8``        per-token symmetric int8 activations after the group FWHT.
* ``q4_0``      Q4_0 block encode / decode.
* ``matmul``    fp64 reference products for the CQ and Q4_0 paths.
* ``fp``        exact fp16 / bf16 rounding helpers.

Parity status: every function here is pinned by a test in ``tests/``
against a closed form, a brute-force search, a textbook value or a figure
the pages print.  Whole-model outputs are out of scope (parity unpinned:
they need trained weights).
"""

from . import fp, hadamard, codebook, cq, a8, q4_0, matmul  # noqa: F401
