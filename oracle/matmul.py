"""fp64 reference products (oracle; test infrastructure only).

Needle .cact/W4A8 article, section 3: weights are [out, in] so each output
row is one reduction stream; decode is a GEMV (activation vector against the
in axis) and prefill a GEMM with the same layout.  The quantizers are
encodings, so the reference is the plain definition on the decoded operands:
y[b, n] = sum_k W_hat[n, k] * x_hat[b, k], in fp64, using the same int8 q and
scale the device consumed (this isolates the matmul from A8 rounding).

``cq_rotated`` is the rotated-domain form the device uses,
y = s_b / G * sum_g norm[n, g] * dot(cb[idx[n, g]], q[b, g]); the two agree
in real arithmetic because H_u H_u = G I (checked by the tests to 1e-12).

``cq_magnitude`` and ``q4_0_magnitude`` are the sums of the absolute values
of the terms of those sums (the rotated-domain terms for CQ).  Rounding a
sum of terms in floating point, whatever the order, errs by at most a small
multiple of the unit roundoff times this magnitude, so it is the scale that
per-element tolerances are stated against.
"""
from __future__ import annotations

import numpy as np

from . import cq as _cq
from .a8 import dequant_a8
from . import q4_0 as _q4


def cq_reference(idx, norm16, group, code, levels, q, s) -> np.ndarray:
    """Plain definition: decode W_hat and x_hat, then an fp64 matmul."""
    w_hat = _cq.decode(idx, norm16, group, code, levels)
    x_hat = dequant_a8(q, s, group)
    return x_hat @ w_hat.T


def cq_rotated(idx, norm16, group, code, levels, q, s) -> np.ndarray:
    """Rotated-domain sum, fp64: s_b/G * sum_g norm * dot(cb[idx], q)."""
    rows, cols = idx.shape
    ng = cols // group
    c = _cq.level_values(idx, code, levels).reshape(rows, ng, group)
    n = np.asarray(norm16, dtype=np.float16).astype(np.float64)
    qq = np.asarray(q, dtype=np.float64).reshape(q.shape[0], ng, group)
    acc = np.einsum("ngi,bgi->bng", c, qq)
    y = np.einsum("bng,ng->bn", acc, n)
    return y * (np.asarray(s, dtype=np.float64)[:, None] / group)


def cq_magnitude(idx, norm16, group, code, levels, q, s) -> np.ndarray:
    """s_b/G * sum_g norm[n, g] * sum_{i in g} |cb[idx[n, i]]| * |q[b, i]|, fp64."""
    rows, cols = idx.shape
    ng = cols // group
    c = np.abs(_cq.level_values(idx, code, levels)).reshape(rows, ng, group)
    n = np.abs(np.asarray(norm16, dtype=np.float16).astype(np.float64))
    qq = np.abs(np.asarray(q, dtype=np.float64)).reshape(q.shape[0], ng, group)
    acc = np.einsum("ngi,bgi->bng", c, qq)
    y = np.einsum("bng,ng->bn", acc, n)
    return y * (np.abs(np.asarray(s, dtype=np.float64))[:, None] / group)


def q4_0_reference(blocks, cols, x) -> np.ndarray:
    """y[b, r] = sum_{k < cols} W_hat[r, k] * x[b, k] in fp64."""
    w_hat = _q4.decode(blocks, cols)
    return np.asarray(x, dtype=np.float64) @ w_hat.T


def q4_0_magnitude(blocks, cols, x) -> np.ndarray:
    """sum_{k < cols} |W_hat[r, k]| * |x[b, k]| in fp64."""
    w_hat = _q4.decode(blocks, cols)
    return np.abs(np.asarray(x, dtype=np.float64)) @ np.abs(w_hat).T


def q4_0_a8_reference(blocks, cols, q, s) -> np.ndarray:
    """Q4_0 weights against int8 activations: y[b, r] = s_b * sum_k W_hat[r, k] * q[b, k],
    fp64 (the plain definition on the decoded operands, x_hat = s * q)."""
    x_hat = np.asarray(q, dtype=np.float64) * np.asarray(s, dtype=np.float64)[:, None]
    return q4_0_reference(blocks, cols, x_hat)


def q4_0_a8_magnitude(blocks, cols, q, s) -> np.ndarray:
    x_hat = np.asarray(q, dtype=np.float64) * np.asarray(s, dtype=np.float64)[:, None]
    return q4_0_magnitude(blocks, cols, x_hat)


def rel_l2(y, ref) -> float:
    """||y - ref||_2 / ||ref||_2 (the tolerance measure); 0-norm ref -> abs."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(y - ref)
    return float(num / den) if den > 0 else float(num)
