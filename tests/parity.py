"""Element-wise parity checks for the fp32 products (shared by the GPU tests).

Every device product is a sum of terms, each formed exactly or with one stated
rounding, accumulated in fp32.  Whatever the order of the additions, such a
sum errs by at most a small multiple of the unit roundoff times the sum of the
absolute values of its terms, which the oracle computes as ``cq_magnitude`` /
``q4_0_magnitude``.  So each output element must satisfy

    |y - y_ref| <= tol * magnitude

with ``tol`` taken from the arithmetic of the path that produced it:

* ``TOL_F32`` (1e-5, about 170 units of fp32 roundoff): the products are exact
  (an fp16 level times an int8 code, a base-3 digit times a code, a 4-bit
  Q4_0 code times its fp16 scale in fp32) or rounded once in fp32 (fp32
  activations on the Q4_0 paths), then summed in fp32 in groups of at most a
  few hundred terms and scaled by fp32 norms.  Rounding errors of that size
  stay below 1e-6 of the magnitude in practice; one weight taken from the
  wrong index moves an element by about 1/K of its magnitude (2.4e-4 at
  K = 4096), far past the bound.
* ``TOL_FOLD`` (2^-11 + 1e-5): the CQ GEMM (and the decode GEMV's route to
  it) rounds level * norm * 2^e to fp16 once per weight, a relative error of
  at most 2^-11 per term, before the same fp32 accumulation.

On top of the element bound each check keeps the tensor-wide relative L2
error at or below 1e-3, the tolerance the benchmark spec states, and an output whose
reference and magnitude are zero (an all-zero weight row) must be exactly 0.
The worst per-row (per output feature) relative error, the largest absolute
error and the largest |y - y_ref| / magnitude are recorded and printed at the
end of the session.
"""
from __future__ import annotations

import numpy as np

from oracle import matmul as omm

TOL_L2 = 1e-3
TOL_F32 = 1e-5
TOL_FOLD = 2.0 ** -11 + TOL_F32

# cq_gemv routing (include/bqm.h, cq_gemv): the matrix-core GEMV takes 2..16
# tokens when cols <= 16384 (3..16 past 4096 columns); past that, more than
# four tokens go to the GEMM kernel and its fp16 fold; the rest run on the
# VALU GEMV.
MMA_MAX_COLS = 16384
MMA_ONE_CHUNK_COLS = 4096

RECORDS: list[dict] = []


def cq_gemv_tol(cols: int, batch: int) -> float:
    """Element tolerance of the cq_gemv / cq_gemv_f32 (with code buffers) route."""
    min_mma = 2 if cols <= MMA_ONE_CHUNK_COLS else 3
    if min_mma <= batch <= 32 and cols <= MMA_MAX_COLS:
        return TOL_F32
    if batch > 4:
        return TOL_FOLD
    return TOL_F32


def check(y, ref, mag, tol: float, label: str = "") -> dict:
    """Assert the element bound and the tensor bound; return (and record) the stats.

    y, ref, mag: [batch, rows] (device result, fp64 oracle, fp64 magnitude)."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    mag = np.asarray(mag, dtype=np.float64)
    assert y.shape == ref.shape == mag.shape, (y.shape, ref.shape, mag.shape)
    assert np.all(np.isfinite(y)), f"{label}: non-finite outputs"
    err = np.abs(y - ref)
    bound = tol * mag
    bad = err > bound
    zero = mag == 0
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(zero, np.where(err > 0, np.inf, 0.0), err / np.where(zero, 1.0, mag))
        rn = np.linalg.norm(ref, axis=0)
        row_rel = np.where(rn > 0, np.linalg.norm(y - ref, axis=0) / np.where(rn > 0, rn, 1.0), 0.0)
    stats = dict(label=label, shape=list(y.shape), tol=tol, rel_l2=omm.rel_l2(y, ref),
                 max_abs=float(err.max()) if err.size else 0.0,
                 max_ratio=float(ratio.max()) if ratio.size else 0.0,
                 worst_row_rel=float(row_rel.max()) if row_rel.size else 0.0,
                 worst_row=int(np.argmax(row_rel)) if row_rel.size else -1)
    RECORDS.append(stats)
    if bad.any():
        b, n = np.argwhere(bad)[0]
        raise AssertionError(
            f"{label}: {int(bad.sum())} of {bad.size} elements past {tol:.3g} x magnitude; first at "
            f"[{b}, {n}]: y {y[b, n]:.9g}, ref {ref[b, n]:.9g}, magnitude {mag[b, n]:.6g} "
            f"(ratio {ratio[b, n]:.3g}); worst row rel {stats['worst_row_rel']:.3g}")
    assert stats["rel_l2"] <= TOL_L2, f"{label}: rel L2 {stats['rel_l2']:.3e}"
    return stats


def check_cq(y, idx, n16, group, code, levels, q, s, tol, label=""):
    ref = omm.cq_reference(idx, n16, group, code, levels, q, s)
    mag = omm.cq_magnitude(idx, n16, group, code, levels, q, s)
    return check(y, ref, mag, tol, label)


def check_q4_0(y, blocks, cols, x, tol=TOL_F32, label=""):
    ref = omm.q4_0_reference(blocks, cols, x)
    mag = omm.q4_0_magnitude(blocks, cols, x)
    return check(y, ref, mag, tol, label)


def summary_lines() -> list[str]:
    if not RECORDS:
        return []
    worst = sorted(RECORDS, key=lambda r: r["max_ratio"] / r["tol"], reverse=True)
    lines = [f"element-wise parity: {len(RECORDS)} product checks; largest |y - ref| / magnitude "
             f"relative to each check's tolerance first:"]
    for r in worst[:12]:
        lines.append(f"  {r['label']:<58} shape {r['shape']}  max|err|/mag {r['max_ratio']:.2e} "
                     f"(tol {r['tol']:.2e})  max|err| {r['max_abs']:.2e}  worst row rel "
                     f"{r['worst_row_rel']:.2e}  rel L2 {r['rel_l2']:.2e}")
    return lines
