"""Pins for the oracle's A8 activations, Q4_0 blocks and reference products (CPU)."""
from __future__ import annotations

import math

import numpy as np
import pytest

from oracle import a8, cq, matmul, q4_0
from oracle import codebook as cb
from tests.conftest import read_golden_rows
from tests.test_oracle_hadamard_fp import parity_hadamard


# ----------------------------------------------------------------------- A8

def test_a8_reconstruction_bound_and_range():
    rng = np.random.default_rng(20)
    x = rng.standard_normal((6, 512)).astype(np.float32)
    q, s = a8.act_quant_a8(x, 128, "fp32")
    assert q.dtype == np.int8 and s.dtype == np.float32
    hu = parity_hadamard(128).astype(np.float64)
    u = (x.astype(np.float64).reshape(6, 4, 128) @ hu.T).reshape(6, 512)   # explicit matrix
    assert np.all(np.abs(q) <= 127)
    for r in range(6):
        k = np.argmax(np.abs(u[r]))
        assert abs(int(q[r, k])) == 127
        # fp32 rounding of u and of the division add at most a few ulp
        assert np.all(np.abs(u[r] - float(s[r]) * q[r]) <= 0.5 * float(s[r]) * (1 + 1e-5) + 1e-4)


def test_a8_zero_row_and_modes_agree():
    rng = np.random.default_rng(21)
    x = rng.standard_normal((4, 256)).astype(np.float32)
    x[2] = 0
    q32, s32 = a8.act_quant_a8(x, 128, "fp32")
    q64, s64 = a8.act_quant_a8(x, 128, "fp64")
    assert np.all(q32[2] == 0) and s32[2] == 1.0
    # the two modes differ only where x_u/s sits within rounding of a .5 boundary
    u = (x.astype(np.float64).reshape(4, 2, 128) @ parity_hadamard(128).T).reshape(4, 256)
    frac = np.abs(np.abs(u / s64[:, None]) % 1.0 - 0.5)
    diff = q32 != q64
    assert np.all(frac[diff] < 1e-4)
    assert diff.mean() < 1e-3


def test_a8_dequant_inverts_rotation():
    """If H_u x is an exact multiple of s, dequant returns x exactly (H_u H_u = G I)."""
    rng = np.random.default_rng(22)
    g = 128
    qv = rng.integers(-127, 128, size=(1, g)).astype(np.float64)
    qv[0, 5] = 127
    s = 0.25
    x = (qv @ parity_hadamard(g).T) * (s / g)          # H_u x = s q exactly
    q, ss = a8.act_quant_a8(x.astype(np.float32), g, "fp64")
    assert np.array_equal(q.astype(np.float64), qv)
    assert np.allclose(a8.dequant_a8(q, ss, g), x, atol=1e-12)


def _sparse(spec: str, n: int = 128) -> np.ndarray:
    v = np.zeros(n, dtype=np.float64)
    for item in spec.split():
        i, val = item.split(":")
        v[int(i)] = float(val)
    return v


def tie_rows():
    """Rows of tests/golden/a8_ties.txt as (x fp32 [128], s, q [128]).

    x = H_u u / 128 with H_u from the bit-parity closed form; every value is
    exact in fp32, so H_u x = u exactly (H_u H_u = 128 I)."""
    g = {r[0].split(":", 1)[0]: r[0].split(":", 1)[1].strip() for r in read_golden_rows("a8_ties.txt")}
    hu = parity_hadamard(128).astype(np.float64)
    out = []
    for r in range(2):
        u = _sparse(g[f"row{r}_u"])
        x64 = (hu @ u) / 128.0
        x32 = x64.astype(np.float32)
        assert np.array_equal(x32.astype(np.float64), x64)
        out.append((x32, float(g[f"row{r}_s"]), _sparse(g[f"row{r}_q"]).astype(np.int64)))
    return out


@pytest.mark.parametrize("mode", ["fp32", "fp64"])
def test_a8_ties_round_half_to_even(mode):
    """Hand-worked codes for exact .5 quotients (half-even; half-away would differ)."""
    for x, s_want, q_want in tie_rows():
        q, s = a8.act_quant_a8(x[None, :], 128, mode)
        assert float(s[0]) == s_want
        assert np.array_equal(q[0].astype(np.int64), q_want)


@pytest.mark.parametrize("mode", ["fp32", "fp64"])
def test_a8_unrotated_ties_and_range(mode):
    """Without the rotation the hand-built rotated values are the activations
    themselves (H of length 1 is the identity): the same hand-worked codes."""
    g = {r[0].split(":", 1)[0]: r[0].split(":", 1)[1].strip() for r in read_golden_rows("a8_ties.txt")}
    for r in range(2):
        x = _sparse(g[f"row{r}_u"]).astype(np.float32)
        q, s = a8.act_quant_a8_unrotated(x[None, :], mode)
        assert float(s[0]) == float(g[f"row{r}_s"])
        assert np.array_equal(q[0].astype(np.int64), _sparse(g[f"row{r}_q"]).astype(np.int64))
    # a zero row, the amax element at +-127, |x - s q| <= s / 2, odd widths
    rng = np.random.default_rng(24)
    x = rng.standard_normal((3, 1092)).astype(np.float32)
    x[1] = 0
    q, s = a8.act_quant_a8_unrotated(x, mode)
    assert np.all(q[1] == 0) and s[1] == 1
    for r in (0, 2):
        k = int(np.argmax(np.abs(x[r])))
        assert abs(int(q[r, k])) == 127
        assert np.all(np.abs(x[r].astype(np.float64) - float(s[r]) * q[r]) <= 0.5 * float(s[r]) * (1 + 1e-6))


# --------------------------------------------------------------------- Q4_0

def test_q4_0_hand_built_block():
    rows = {r[0].split(":")[0]: r[0].split(":")[1] for r in read_golden_rows("q4_0_block.txt")}
    w = np.array([[float(v) for v in rows["weights"].split()]], dtype=np.float32)
    want = np.array([int(v, 16) for v in rows["bytes"].split()], dtype=np.uint8)
    blk = q4_0.encode(w)
    assert blk.shape == (1, 1, 18)
    assert np.array_equal(blk[0, 0], want)
    zero = q4_0.encode(np.zeros((1, 32), dtype=np.float32))
    assert np.array_equal(zero[0, 0], np.array([int(v, 16) for v in rows["zero_bytes"].split()], dtype=np.uint8))
    nib = [int(v) for v in rows["nibbles"].split()]
    assert np.array_equal(q4_0.decode(blk, 32)[0], (np.array(nib) - 8) * 2.0)


def test_q4_0_roundtrip_bound_and_padding():
    rng = np.random.default_rng(23)
    w = (0.02 * rng.standard_normal((9, 312))).astype(np.float32)
    blk = q4_0.encode(w)
    assert blk.shape == (9, 10, 18)
    wh = q4_0.decode(blk, 312)
    padded = np.zeros((9, 320), dtype=np.float32)
    padded[:, :312] = w
    d = np.max(np.abs(padded.reshape(9, 10, 32)), axis=-1) / 8.0
    pb = padded.reshape(9, 10, 32).astype(np.float64)
    err = np.abs(pb - np.pad(wh, ((0, 0), (0, 8))).reshape(9, 10, 32))
    dd = np.broadcast_to(d[..., None].astype(np.float64), err.shape)
    clipped = pb / dd > 7.5                    # the +amax element maps to 8, clipped to 7
    # |w - q d| <= d/2, plus |q| * |d - fp16(d)| <= 8 * 2^-11 d from the stored scale
    assert np.all(err[~clipped] <= dd[~clipped] * (0.5 + 2.0 ** -8) + 1e-12)
    assert np.all(err[clipped] <= dd[clipped] * (1.0 + 2.0 ** -8) + 1e-12)
    assert clipped.sum() > 0
    # the last block holds 24 real columns and 8 padding nibbles equal to 8
    last = blk[:, 9, 2:]
    assert np.all((last[:, 12:] == 0x88))
    full = q4_0.decode(blk, 320)
    assert np.all(full[:, 312:] == 0)
    # every code in [-8, 7]
    nib = np.concatenate([blk[..., 2:] & 0xF, blk[..., 2:] >> 4], axis=-1)
    assert nib.min() >= 0 and nib.max() <= 15


def test_q4_0_sizes_reproduce_minueza_files():
    """Q4_0 at 18 B per 32 padded weights reproduces the page's 12.58 / 18.07 MB
    images (KMCU v1: 128 B header, 48 B records, 64-aligned data, f32 norms)."""
    g = {r[0].split(":")[0]: float(r[0].split(":")[1]) for r in read_golden_rows("minueza_sizes.txt")}
    dim, ffn, vocab, layers = 312, 1092, 32002, 10
    mats = [(dim, dim), (104, dim), (104, dim), (dim, dim), (ffn, dim), (ffn, dim), (dim, ffn)]

    def image(untied: bool):
        tensors = [("q4", vocab, dim)]
        for _ in range(layers):
            tensors.append(("f32", 1, dim))
            tensors += [("q4", r, c) for r, c in mats[:4]]
            tensors.append(("f32", 1, dim))
            tensors += [("q4", r, c) for r, c in mats[4:]]
        tensors.append(("f32", 1, dim))
        if untied:
            tensors.append(("q4", vocab, dim))
        off = 128 + 48 * len(tensors)
        params = 0
        for kind, r, c in tensors:
            off = (off + 63) // 64 * 64
            off += q4_0.nbytes(r, c) if kind == "q4" else 4 * r * c
            params += r * c
        return off, params

    tb, tp = image(False)
    ub, up = image(True)
    assert round(tp / 1e6, 2) == g["tied_params_millions"]
    assert round(up / 1e6, 2) == g["untied_params_millions"]
    assert round(tb / 2 ** 20, 2) == g["tied_mib"]
    assert round(ub / 2 ** 20, 2) == g["untied_mib"]


# ----------------------------------------------------------------- products

def _h_entry(i, j):
    return -1.0 if bin(i & j).count("1") % 2 else 1.0


def brute_force_cq(idx, n16, g, code, levels, q, s):
    """Scalar triple loop with H_u entries from the bit-parity closed form."""
    rows, cols = idx.shape
    lv = np.concatenate([levels.astype(np.float64), np.zeros(16)])
    m = q.shape[0]
    y = np.zeros((m, rows))
    for b in range(m):
        for n in range(rows):
            tot = 0.0
            for gs in range(0, cols, g):
                for k in range(g):
                    wk = sum(_h_entry(k, j) * lv[idx[n, gs + j]] for j in range(g)) * float(n16[n, gs // g]) / g
                    xk = sum(_h_entry(k, j) * float(q[b, gs + j]) for j in range(g)) * float(s[b]) / g
                    tot += wk * xk
            y[b, n] = tot
    return y


@pytest.mark.parametrize("m,rows,g,cols", [(1, 1, 8, 8), (2, 2, 16, 16), (1, 3, 128, 128)])
def test_cq_reference_brute_force(m, rows, g, cols):
    rng = np.random.default_rng(30 + g)
    for code in (cq.B4, cq.TERNARY, cq.BINARY):
        lv = cb.analytic_levels(code) if code != cq.B4 else cb.shipped_table(cb.lloyd_max_quadrature(16))
        w = (0.02 * rng.standard_normal((rows, cols))).astype(np.float32)
        x = rng.standard_normal((m, cols)).astype(np.float32)
        idx, n16 = cq.encode(w, g, code, lv)
        q, s = a8.act_quant_a8(x, g, "fp32")
        ref = brute_force_cq(idx, n16, g, code, lv, q, s)
        assert np.max(np.abs(matmul.cq_reference(idx, n16, g, code, lv, q, s) - ref)) < 1e-12 * max(1, np.abs(ref).max())
        assert np.max(np.abs(matmul.cq_rotated(idx, n16, g, code, lv, q, s) - ref)) < 1e-12 * max(1, np.abs(ref).max())


@pytest.mark.parametrize("code", [1, 2, 3, 4, 5])
def test_rotated_identity(code, codebooks):
    rng = np.random.default_rng(40 + code)
    w = (0.02 * rng.standard_normal((48, 512))).astype(np.float32)
    w[7] *= 8
    w[9, :128] = 0
    x = rng.standard_normal((3, 512)).astype(np.float32)
    lv = cq.levels_for(code, codebooks)
    idx, n16 = cq.encode(w, 128, code, lv)
    q, s = a8.act_quant_a8(x, 128, "fp32")
    y_ref = matmul.cq_reference(idx, n16, 128, code, lv, q, s)
    y_rot = matmul.cq_rotated(idx, n16, 128, code, lv, q, s)
    assert matmul.rel_l2(y_rot, y_ref) < 1e-12


def test_q4_0_reference_brute_force():
    rng = np.random.default_rng(50)
    w = (0.02 * rng.standard_normal((3, 40))).astype(np.float32)
    x = rng.standard_normal((2, 40)).astype(np.float32)
    blk = q4_0.encode(w)
    ref = np.zeros((2, 3))
    for b in range(2):
        for r in range(3):
            for k in range(40):
                byte = blk[r, k // 32, 2 + (k % 32) // 2]
                nib = (byte >> 4) if k % 2 else (byte & 0xF)
                d = float(blk[r, k // 32, 0:2].view(np.float16)[0])
                ref[b, r] += (int(nib) - 8) * d * float(x[b, k])
    assert np.max(np.abs(matmul.q4_0_reference(blk, 40, x) - ref)) < 1e-15


def test_rel_l2():
    assert matmul.rel_l2([1.0, 2.0], [1.0, 2.0]) == 0.0
    assert math.isclose(matmul.rel_l2([1.0, 0.0], [0.0, 0.0]), 1.0)


@pytest.mark.parametrize("code", [1, 4, 5])
def test_cq_magnitude_bounds_and_equality(code, codebooks):
    """The magnitude is >= |y| for every element (triangle inequality) and equals
    the product itself when every term is non-negative (non-negative codes and
    only non-negative levels), where the plain definition is pinned by brute force."""
    rng = np.random.default_rng(60 + code)
    w = (0.02 * rng.standard_normal((20, 256))).astype(np.float32)
    w[3] *= 1e-4
    x = rng.standard_normal((3, 256)).astype(np.float32)
    lv = cq.levels_for(code, codebooks)
    idx, n16 = cq.encode(w, 128, code, lv)
    q, s = a8.act_quant_a8(x, 128, "fp32")
    y = matmul.cq_reference(idx, n16, 128, code, lv, q, s)
    mag = matmul.cq_magnitude(idx, n16, 128, code, lv, q, s)
    assert np.all(np.abs(y) <= mag * (1 + 1e-12))
    assert np.all(mag > 0)
    # every index at the largest (positive) level, codes |q|: all terms >= 0
    top = np.full_like(idx, int(np.argmax(lv)))
    qa = np.abs(q.astype(np.int64)).astype(np.int8)
    yp = matmul.cq_reference(top, n16, 128, code, lv, qa, s)
    mp = matmul.cq_magnitude(top, n16, 128, code, lv, qa, s)
    assert np.allclose(mp, yp, rtol=1e-12, atol=0)
    # signs do not matter to the magnitude
    qf = qa.copy()
    qf[:, ::3] = -qf[:, ::3]
    assert np.array_equal(matmul.cq_magnitude(top, n16, 128, code, lv, qf, s), mp)


def test_q4_0_magnitude_bounds_and_equality():
    rng = np.random.default_rng(61)
    w = (0.02 * rng.standard_normal((7, 70))).astype(np.float32)
    x = rng.standard_normal((2, 70)).astype(np.float32)
    blk = q4_0.encode(w)
    y = matmul.q4_0_reference(blk, 70, x)
    mag = matmul.q4_0_magnitude(blk, 70, x)
    assert np.all(np.abs(y) <= mag * (1 + 1e-12)) and np.all(mag > 0)
    wp = np.abs(w)
    blp = q4_0.encode(wp)
    xp = np.abs(x)
    assert np.allclose(matmul.q4_0_magnitude(blp, 70, xp), matmul.q4_0_reference(blp, 70, xp), rtol=1e-12)


def test_q4_0_a8_reference_brute_force():
    """Q4_0 weights x int8 codes: a scalar loop over the blocks' bytes."""
    rng = np.random.default_rng(51)
    w = (0.02 * rng.standard_normal((3, 45))).astype(np.float32)
    x = rng.standard_normal((2, 45)).astype(np.float32)
    blk = q4_0.encode(w)
    q, s = a8.act_quant_a8_unrotated(x)
    ref = np.zeros((2, 3))
    for b in range(2):
        for r in range(3):
            for k in range(45):
                byte = blk[r, k // 32, 2 + (k % 32) // 2]
                nib = (byte >> 4) if k % 2 else (byte & 0xF)
                d = float(blk[r, k // 32, 0:2].view(np.float16)[0])
                ref[b, r] += (int(nib) - 8) * d * int(q[b, k])
            ref[b, r] *= float(s[b])
    assert np.max(np.abs(matmul.q4_0_a8_reference(blk, 45, q, s) - ref)) < 1e-15 * max(1.0, np.abs(ref).max())
    mag = matmul.q4_0_a8_magnitude(blk, 45, q, s)
    assert np.all(np.abs(ref) <= mag * (1 + 1e-12))
