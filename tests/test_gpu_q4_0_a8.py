"""GPU parity of the int8-activation (A8) Q4_0 path against the oracle.

The unrotated per-token codes (act_fwht_quant_a8 with group 1) are compared
bit for bit, including a row of exact .5 quotients; the Q4_0 x int8 products
(q4_0_gemv_a8, q4_0_gemm_a8) element by element, |y - y_ref| <= 1e-5 x the
magnitude (exact int32 block sums, one fp32 rounding per block term and fp32
accumulation), and rel-L2 <= 1e-3.  Widths include rows that are not a
multiple of 32 (padding) or of 4 (unaligned code rows)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from bit_quantized_matmul_amd import binding as B
from bit_quantized_matmul_amd import inputs
from oracle import a8 as oa8
from oracle import matmul as omm
from oracle import q4_0 as oq4
from tests import parity as P
from tests.test_oracle_a8_q4_0_matmul import _sparse
from tests.conftest import read_golden_rows

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def check(y, blk, cols, q, s, label):
    ref = omm.q4_0_a8_reference(blk, cols, q, s)
    mag = omm.q4_0_a8_magnitude(blk, cols, q, s)
    return P.check(y, ref, mag, P.TOL_F32, label)


@pytest.mark.parametrize("m,k", [(1, 312), (3, 1092), (5, 33), (2, 4096), (1, 20000), (512, 312), (4, 1), (2, 65536)])
def test_act_quant_a8_unrotated_bit_exact(m, k):
    rng = np.random.default_rng(1600 + m + k)
    x = inputs.activations(rng, m, k)
    if m > 1:
        x[1] = 0.0                                        # zero row: s = 1, q = 0
    if m > 2 and k >= 128:
        g = {r[0].split(":", 1)[0]: r[0].split(":", 1)[1].strip() for r in read_golden_rows("a8_ties.txt")}
        x[2] = 0.0
        x[2, :128] = _sparse(g["row0_u"]).astype(np.float32)   # exact .5 quotients
    q_ref, s_ref = oa8.act_quant_a8_unrotated(x, "fp32")
    q, s = B.act_fwht_quant_a8(dev(x), group=1)
    assert np.array_equal(host(q), q_ref)
    assert np.array_equal(host(s).view(np.uint32), s_ref.view(np.uint32))


def case(rng, rows, cols, batch, mixed=False):
    w = (inputs.weight_matrix_mixed(rng, rows, cols, group=32) if mixed
         else inputs.weight_matrix(rng, rows, cols))
    x = inputs.activations(rng, batch, cols)
    blk = oq4.encode(w)
    q, s = oa8.act_quant_a8_unrotated(x, "fp32")
    return blk, q, s


@pytest.mark.parametrize("rows,cols,batch", [(312, 312, 1), (104, 312, 1), (1092, 312, 1), (312, 1092, 1),
                                             (300, 40, 3), (7, 1000, 16), (33, 33, 2), (5, 1, 1),
                                             (64, 2050, 4), (32002, 312, 1), (257, 101, 5)])
def test_q4_0_gemv_a8_parity(rows, cols, batch):
    rng = np.random.default_rng(1610 + rows + cols + batch)
    blk, q, s = case(rng, rows, cols, batch)
    y = host(B.q4_0_gemv_a8(dev(blk.ravel()), rows, cols, dev(q), dev(s)))
    check(y, blk, cols, q, s, f"q4_0_gemv_a8 {rows}x{cols} b{batch}")


@pytest.mark.parametrize("rows,cols,m", [(312, 312, 37), (104, 312, 512), (1092, 312, 64), (312, 1092, 100),
                                         (32002, 312, 130), (70, 33, 65), (129, 101, 3), (1, 1, 1), (5, 64, 1),
                                         (300, 4096, 40), (1, 96, 5), (3, 32, 7), (7, 160, 33), (9, 35, 3)])
def test_q4_0_gemm_a8_parity(rows, cols, m):
    rng = np.random.default_rng(1620 + rows + cols + m)
    blk, q, s = case(rng, rows, cols, m)
    db, dq, ds = dev(blk.ravel()), dev(q), dev(s)
    y = host(B.q4_0_gemm_a8(db, rows, cols, dq, ds))
    check(y, blk, cols, q, s, f"q4_0_gemm_a8 m{m} {rows}x{cols}")
    # a token's row equals the GEMV's sum up to fp32 order
    g = host(B.q4_0_gemv_a8(db, rows, cols, dq[:1], ds[:1]))
    assert np.all(np.abs(y[:1] - g) <= 2 * P.TOL_F32 * omm.q4_0_a8_magnitude(blk, cols, q[:1], s[:1]))


@pytest.mark.parametrize("entry,rows,cols,n", [("gemv", 60, 312, 1), ("gemv", 60, 1092, 3),
                                               ("gemm", 60, 312, 37), ("gemm", 300, 1092, 100)])
def test_q4_0_a8_mixed_scale_rows(entry, rows, cols, n):
    rng = np.random.default_rng(1630 + rows + cols + n)
    blk, q, s = case(rng, rows, cols, n, mixed=True)
    fn = B.q4_0_gemv_a8 if entry == "gemv" else B.q4_0_gemm_a8
    y = host(fn(dev(blk.ravel()), rows, cols, dev(q), dev(s)))
    assert np.all(y[:, rows // 2] == 0.0)
    check(y, blk, cols, q, s, f"mixed q4_0_{entry}_a8 {rows}x{cols} n{n}")


# the fused entry (codes formed in the launch): token slices of 4, 2 and 1,
# widths of 1..1706 blocks (ragged, cols % 4 != 0), a zero token, rows from 1
# to the tied head; y, the codes and the scales equal the two-launch path's
# bit for bit, and y the oracle's within the bound
@pytest.mark.parametrize("rows,cols,batch", [(312, 312, 1), (104, 312, 3), (1092, 312, 16), (312, 1092, 7),
                                             (5, 33, 2), (1, 1, 1), (32002, 312, 1), (64, 14336, 5),
                                             (40, 54592, 1), (257, 101, 4), (33, 4097, 6)])
def test_q4_0_gemv_a8_f32_matches_two_launches(rows, cols, batch):
    rng = np.random.default_rng(1650 + rows + cols + batch)
    w = inputs.weight_matrix(rng, rows, cols)
    x = inputs.activations(rng, batch, cols)
    if batch > 1:
        x[1] = 0.0                                        # zero token: s = 1, q = 0, y = 0
    blk = oq4.encode(w)
    db, dx = dev(blk.ravel()), dev(x)
    q_out = torch.empty((batch, cols), dtype=torch.int8, device=DEV)
    s_out = torch.empty((batch,), dtype=torch.float32, device=DEV)
    y = host(B.q4_0_gemv_a8_f32(db, rows, cols, dx, q_out=q_out, scale_out=s_out))
    q, s = B.act_fwht_quant_a8(dx, group=1)
    y2 = host(B.q4_0_gemv_a8(db, rows, cols, q, s))
    assert np.array_equal(host(q_out), host(q))
    assert np.array_equal(host(s_out).view(np.uint32), host(s).view(np.uint32))
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))
    q_ref, s_ref = oa8.act_quant_a8_unrotated(x, "fp32")
    assert np.array_equal(host(q_out), q_ref)
    if batch > 1:
        assert np.all(y[1] == 0.0)
    sel = np.arange(rows) if rows <= 2048 else np.sort(rng.choice(rows, 64, replace=False))
    check(y[:, sel], blk[sel], cols, q_ref, s_ref, f"q4_0_gemv_a8_f32 {rows}x{cols} b{batch}")


def test_q4_0_gemv_a8_f32_ties():
    """Quotients that are exact halves take the correctly rounded division's
    tie rule (the codes of the hand-worked tie row), in the fused launch."""
    g = {r[0].split(":", 1)[0]: r[0].split(":", 1)[1].strip() for r in read_golden_rows("a8_ties.txt")}
    x = np.zeros((1, 128), dtype=np.float32)
    x[0] = _sparse(g["row0_u"]).astype(np.float32)
    rng = np.random.default_rng(1660)
    blk = oq4.encode(inputs.weight_matrix(rng, 40, 128))
    q_out = torch.empty((1, 128), dtype=torch.int8, device=DEV)
    B.q4_0_gemv_a8_f32(dev(blk.ravel()), 40, 128, dev(x), q_out=q_out)
    q_ref, _ = oa8.act_quant_a8_unrotated(x, "fp32")
    assert np.array_equal(host(q_out), q_ref)


def test_q4_0_a8_device_codes_end_to_end():
    """Device A8 codes feed the device products: the whole int8 path on the
    Minueza head shape at 64 tokens against the oracle's codes and product."""
    rng = np.random.default_rng(1640)
    rows, cols, m = 32002, 312, 64
    w = inputs.weight_matrix(rng, rows, cols)
    x = inputs.activations(rng, m, cols)
    blocks = B.q4_0_pack(dev(w))
    q, s = B.act_fwht_quant_a8(dev(x), group=1)
    y = host(B.q4_0_gemm_a8(blocks, rows, cols, q, s))
    q_ref, s_ref = oa8.act_quant_a8_unrotated(x, "fp32")
    assert np.array_equal(host(q), q_ref)
    sel = np.sort(rng.choice(rows, 48, replace=False))
    blk = oq4.encode(w[sel])
    assert np.array_equal(host(blocks).reshape(rows, -1, 18)[sel], blk)
    check(y[:, sel], blk, cols, q_ref, s_ref, "q4_0 A8 end to end (sampled rows)")
