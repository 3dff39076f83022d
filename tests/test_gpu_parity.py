"""GPU parity: every C-ABI entry point against the CPU oracle.

Bit-exact for byte / integer results (packed blobs, Q4_0 blocks, int8
activations and their scales, the codebook fit).  The fp32 products are
checked element by element against the fp64 oracle: |y - y_ref| <= tol x the
oracle's magnitude (the sum of the absolute values of the terms), with tol
from each path's arithmetic, and the tensor's relative L2 error <= 1e-3 (the
tolerance the benchmark spec states); see tests/parity.py.  Inputs are seeded; products
use the oracle's own packed weights and int8 activations, so the device
encoders and the device products are checked independently.  Matrices with
rows at scales 1, 1e-3, 1e-4 and 1e-6, a row of mixed-scale groups and an
all-zero row run through every product route.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from bit_quantized_matmul_amd import binding as B
from bit_quantized_matmul_amd import inputs
from oracle import a8 as oa8
from oracle import codebook as ocb
from oracle import cq as ocq
from oracle import matmul as omm
from oracle import q4_0 as oq4
from tests import parity as P
from tests.conftest import read_golden_rows

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def weights(rng, rows, cols, outliers=True, zero_group=True):
    w = inputs.weight_matrix(rng, rows, cols, outliers=outliers)
    if zero_group and rows > 2:
        w[1, :128] = 0.0                                  # an all-zero group
    return w


def levels(code, codebooks):
    return ocq.levels_for(code, codebooks)


def host_codebook(code, codebooks):
    return None if code in (ocq.BINARY, ocq.TERNARY, ocq.TERNARY_B3) else codebooks[code]


# ------------------------------------------------------------------ encoders

def a8_tie_row():
    """The first hand-built row of tests/golden/a8_ties.txt as fp32 activations:
    x = H_u u / 128 (exact in fp32), so that H_u x = u exactly and u / s = u."""
    from tests.test_oracle_a8_q4_0_matmul import tie_rows
    return tie_rows()[0][0]


@pytest.mark.parametrize("m,k", [(1, 128), (3, 512), (2, 1024), (4, 2048), (5, 4096), (3, 8192), (2, 14336),
                                 (2, 24576), (1, 65536), (512, 4096)])
def test_act_quant_bit_exact(m, k):
    rng = np.random.default_rng(100 + m + k)
    x = inputs.activations(rng, m, k)
    if m > 1:
        x[1] = 0.0                                          # zero row -> s = 1, q = 0
    x[0, :7] *= 50.0                                        # a few large entries
    if m > 2:
        x[2, :128] = a8_tie_row()                            # exact .5 quotients (half-even)
        x[2, 128:] = 0.0
    q_ref, s_ref = oa8.act_quant_a8(x, 128, "fp32")
    q, s = B.act_fwht_quant_a8(dev(x))
    assert np.array_equal(host(q), q_ref)
    assert np.array_equal(host(s).view(np.uint32), s_ref.view(np.uint32))


@pytest.mark.parametrize("code", [1, 2, 3, 4, 5, 6])
@pytest.mark.parametrize("rows,cols", [(300, 512), (3, 128), (65, 1024)])
def test_cq_pack_bit_exact(code, rows, cols, codebooks):
    rng = np.random.default_rng(200 + code + rows)
    w = weights(rng, rows, cols)
    lv = levels(code, codebooks)
    idx, n16 = ocq.encode(w, 128, code, lv)
    ref = ocq.make_blob(idx, n16, 128, code)
    lay = B.cq_pack_info(rows, cols, 128, code)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    blob = torch.full((lay.total_bytes,), 0xA5, dtype=torch.uint8, device=DEV)
    B.cq_pack(dev(w), lay, host_codebook(code, codebooks), blob=blob, status=status)
    got = host(blob)
    assert int(host(status)[0]) == 0
    if not np.array_equal(got, ref):
        gi, gn = ocq.split_blob(got, rows, cols, 128, code)
        bad_idx = np.argwhere(gi != idx)
        bad_n = np.argwhere(gn.view(np.uint16) != n16.view(np.uint16))
        pytest.fail(f"blob differs: {len(bad_idx)} indices (first {bad_idx[:5].tolist()}), "
                    f"{len(bad_n)} norms (first {bad_n[:5].tolist()})")


def test_cq_pack_reports_overflow_and_nonfinite(codebooks):
    w = np.zeros((2, 128), dtype=np.float32)
    w[0] = 1.0e4                                            # norm 1.13e5 > fp16 max
    w[1, 5] = np.inf
    lay = B.cq_pack_info(2, 128, 128, 4)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    B.cq_pack(dev(w), lay, codebooks[4], status=status)
    st = int(host(status)[0])
    assert st & B.STATUS_NORM_OVERFLOW and st & B.STATUS_NONFINITE


@pytest.mark.parametrize("rows,cols", [(300, 312), (17, 1092), (5, 40), (1, 32), (2, 33)])
def test_q4_0_pack_bit_exact(rows, cols):
    rng = np.random.default_rng(300 + rows + cols)
    w = inputs.weight_matrix(rng, rows, cols)
    if rows > 1:
        w[1, :32] = 0.0                                     # zero block -> d = 1
    ref = oq4.encode(w).ravel()
    got = host(B.q4_0_pack(dev(w)))
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("levels_n", [4, 8, 16])
def test_codebook_fit_bit_exact(levels_n, gaussian400k, raw_fits):
    bits = {4: 2, 8: 3, 16: 4}[levels_n]
    table, raw = B.cq_codebook_fit(dev(gaussian400k), levels_n, 200)
    assert np.array_equal(host(raw), raw_fits[bits])
    assert np.array_equal(host(table), ocb.shipped_table(raw_fits[bits]))


# ------------------------------------------------------------------ products

def oracle_case(rng, rows, cols, code, batch, codebooks):
    w = weights(rng, rows, cols)
    x = inputs.activations(rng, batch, cols)
    lv = levels(code, codebooks)
    idx, n16 = ocq.encode(w, 128, code, lv)
    blob = ocq.make_blob(idx, n16, 128, code)
    q, s = oa8.act_quant_a8(x, 128, "fp32")
    return lv, idx, n16, blob, q, s


@pytest.mark.parametrize("code", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("rows,cols,batch", [(300, 512, 1), (130, 4096, 1), (67, 14336, 1),
                                             (300, 512, 3), (70, 4096, 4), (33, 1024, 16),
                                             (5, 128, 2), (1, 256, 1),
                                             # 2..16 tokens: one matrix-core pass; K eighths
                                             # without groups (128, 384), 1..8 row blocks
                                             # per workgroup with ragged ends; past 4096
                                             # columns K in chunks (5120 x 8, x 3) and the
                                             # VALU GEMV for 2 tokens (5120 x 2); past 16384
                                             # columns more than 4 tokens take the GEMM
                                             # kernel (20480 x 5, 36864 x 8); one row block
                                             # a CU, 64+ groups a row and more than 8
                                             # tokens split K in two halves (8192: one chunk
                                             # each; 8320: 32 and 33 groups, 3 row blocks;
                                             # 12288; 16384 with 2 row blocks; 8192 at 6
                                             # tokens: no split)
                                             (77, 128, 9), (1000, 384, 5), (300, 4096, 12),
                                             (5000, 512, 6), (9000, 256, 16), (40000, 128, 7),
                                             (40, 5120, 8), (40, 5120, 3), (40, 5120, 2),
                                             (20, 20480, 5), (9, 36864, 8),
                                             # 17..32 tokens: two 16-token halves (a
                                             # ragged second half, 4 row blocks, K in
                                             # chunks), past 16384 columns the GEMM
                                             (300, 4096, 24), (9000, 512, 32), (20, 20480, 24),
                                             (300, 8192, 10), (33, 8320, 9), (1000, 12288, 16), (17, 16384, 12),
                                             (300, 8192, 6)])
def test_cq_gemv_parity(code, rows, cols, batch, codebooks):
    rng = np.random.default_rng(400 + code * 7 + rows + batch)
    lv, idx, n16, blob, q, s = oracle_case(rng, rows, cols, code, batch, codebooks)
    lay = B.cq_pack_info(rows, cols, 128, code)
    y = host(B.cq_gemv(dev(blob), lay, host_codebook(code, codebooks), dev(q), dev(s)))
    P.check_cq(y, idx, n16, 128, code, lv, q, s, P.cq_gemv_tol(cols, batch),
               f"cq_gemv code {code} {rows}x{cols} b{batch}")


@pytest.mark.parametrize("code", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("rows,cols,batch", [(300, 512, 1), (130, 4096, 1), (67, 14336, 1),
                                             (1024, 4096, 1), (70, 4096, 4), (33, 1024, 16),
                                             (5, 128, 2), (1, 256, 1), (200, 4096, 3),
                                             (129, 640, 16), (300, 4096, 7), (50, 5120, 3),
                                             # one token past 8192 columns: 8-element
                                             # segments (8320: 1040 of them, 16384: two a thread)
                                             (40, 8320, 1), (9, 16384, 1)])
def test_cq_gemv_f32_fused_matches_two_step(code, rows, cols, batch, codebooks):
    """One-launch A8 + GEMV: the codes and scales equal the oracle's bit for bit and y
    equals the two-launch path (act_fwht_quant_a8, then cq_gemv) bit for bit."""
    rng = np.random.default_rng(450 + code * 13 + rows + batch)
    w = weights(rng, rows, cols)
    x = inputs.activations(rng, batch, cols)
    if batch > 1:
        x[1] = 0.0                                       # zero token: s = 1, codes 0
    lv = levels(code, codebooks)
    idx, n16 = ocq.encode(w, 128, code, lv)
    blob = dev(ocq.make_blob(idx, n16, 128, code))
    lay = B.cq_pack_info(rows, cols, 128, code)
    cb = host_codebook(code, codebooks)
    dx = dev(x)
    q_out = torch.empty((batch, cols), dtype=torch.int8, device=DEV)
    s_out = torch.empty((batch,), dtype=torch.float32, device=DEV)
    y1 = host(B.cq_gemv_f32(blob, lay, cb, dx, q_out=q_out, scale_out=s_out))
    q, s = B.act_fwht_quant_a8(dx)
    y2 = host(B.cq_gemv(blob, lay, cb, q, s))
    q_ref, s_ref = oa8.act_quant_a8(x, 128, "fp32")
    assert np.array_equal(host(q_out), q_ref)
    assert np.array_equal(host(s_out).view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    P.check_cq(y1, idx, n16, 128, code, lv, q_ref, s_ref, P.cq_gemv_tol(cols, batch),
               f"cq_gemv_f32 code {code} {rows}x{cols} b{batch}")


# Base-3 ternary, one token: one group slot a lane (up to 64 groups: 1, 3, 5, 32,
# 64 groups, 64 / 16 / 8 / 2 / 1 rows a wave pass) and two (65, 112 and 128
# groups), odd group counts (rows start 2 bytes off a word), ragged passes
@pytest.mark.parametrize("rows,cols", [(300, 512), (5, 128), (1000, 384), (9, 640), (130, 4096),
                                       (77, 8192), (33, 8320), (67, 14336), (50, 16384), (1, 256),
                                       (257, 1152)])
def test_cq_gemv_ternary_b3_parity(rows, cols, codebooks):
    rng = np.random.default_rng(480 + rows + cols)
    lv, idx, n16, blob, q, s = oracle_case(rng, rows, cols, ocq.TERNARY_B3, 1, codebooks)
    lay = B.cq_pack_info(rows, cols, 128, ocq.TERNARY_B3)
    y = host(B.cq_gemv(dev(blob), lay, None, dev(q), dev(s)))
    P.check_cq(y, idx, n16, 128, ocq.TERNARY_B3, lv, q, s, P.TOL_F32, f"cq_gemv base-3 {rows}x{cols} b1")
    # the same weights packed in 2-bit fields give the same product up to fp32 order
    lay5 = B.cq_pack_info(rows, cols, 128, ocq.TERNARY)
    y5 = host(B.cq_gemv(dev(ocq.make_blob(idx, n16, 128, ocq.TERNARY)), lay5, None, dev(q), dev(s)))
    mag = omm.cq_magnitude(idx, n16, 128, ocq.TERNARY_B3, lv, q, s)
    assert np.all(np.abs(y - y5) <= 2 * P.TOL_F32 * mag)
    # fp32 activations: A8 into the code buffers, then the same product, bit for bit
    x = inputs.activations(rng, 1, cols)
    q_out = torch.empty((1, cols), dtype=torch.int8, device=DEV)
    s_out = torch.empty((1,), dtype=torch.float32, device=DEV)
    y1 = host(B.cq_gemv_f32(dev(blob), lay, None, dev(x), q_out=q_out, scale_out=s_out))
    y2 = host(B.cq_gemv(dev(blob), lay, None, q_out, s_out))
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))


@pytest.mark.parametrize("code", [1, 4, 5])
@pytest.mark.parametrize("rows,cols,batch", [(90, 1024, 3), (33, 4096, 16)])
def test_cq_gemv_f32_fused_without_code_buffers(code, rows, cols, batch, codebooks):
    """Several tokens with no q_out / scale_out: the fused launches per 4 tokens."""
    rng = np.random.default_rng(470 + code + rows + batch)
    w = weights(rng, rows, cols)
    x = inputs.activations(rng, batch, cols)
    lv = levels(code, codebooks)
    idx, n16 = ocq.encode(w, 128, code, lv)
    blob = dev(ocq.make_blob(idx, n16, 128, code))
    lay = B.cq_pack_info(rows, cols, 128, code)
    y = host(B.cq_gemv_f32(blob, lay, host_codebook(code, codebooks), dev(x)))
    q_ref, s_ref = oa8.act_quant_a8(x, 128, "fp32")
    P.check_cq(y, idx, n16, 128, code, lv, q_ref, s_ref, P.TOL_F32,
               f"cq_gemv_f32 fused code {code} {rows}x{cols} b{batch}")


@pytest.mark.parametrize("code", [1, 2, 3, 4, 5])
# cols 1024 / 2048 / 3072: group counts that are multiples of 8 (norms 8 groups
# to a load, 1-3 rounds, tiles starting their walk at different rounds);
# 1152: 9 groups, the per-group norm path past one round
@pytest.mark.parametrize("m,rows,cols", [(37, 300, 512), (128, 256, 1024), (1, 100, 128),
                                         (200, 130, 384), (257, 64, 256), (70, 200, 2048),
                                         (130, 96, 3072), (33, 50, 1152)])
def test_cq_gemm_parity(code, m, rows, cols, codebooks):
    rng = np.random.default_rng(500 + code * 11 + m + rows)
    lv, idx, n16, blob, q, s = oracle_case(rng, rows, cols, code, m, codebooks)
    lay = B.cq_pack_info(rows, cols, 128, code)
    y = host(B.cq_gemm(dev(blob), lay, host_codebook(code, codebooks), dev(q), dev(s)))
    P.check_cq(y, idx, n16, 128, code, lv, q, s, P.TOL_FOLD, f"cq_gemm code {code} m{m} {rows}x{cols}")


# One shape per prefill tile, compared element by element.  The launch takes
# the largest tile whose count reaches 7/8 of the CUs; on a 256-CU MI355X,
# 500 tokens (ragged m-tiles) with 3600 rows take 64x128, with 7300 rows
# 128x128, with 14100 rows 128x256 (every one with a ragged n-tile).  K of 8
# groups loads the norms 8 to a load, K of 9 groups one by one.
@pytest.mark.parametrize("rows", [3600, 7300, 14100])
@pytest.mark.parametrize("cols", [1024, 1152])
def test_cq_gemm_every_tile(rows, cols, codebooks):
    rng = np.random.default_rng(1500 + rows + cols)
    lv, idx, n16, blob, q, s = oracle_case(rng, rows, cols, 4, 500, codebooks)
    lay = B.cq_pack_info(rows, cols, 128, 4)
    y = host(B.cq_gemm(dev(blob), lay, host_codebook(4, codebooks), dev(q), dev(s)))
    P.check_cq(y, idx, n16, 128, 4, lv, q, s, P.TOL_FOLD, f"cq_gemm tile case m500 {rows}x{cols}")


# Up to 32 tokens cq_gemm runs the batched decode kernel in one launch (two
# 16-token halves on the same weight fragments; exact fp16 products), up to 64
# in launches of 32 where the GEMM's tiles would leave CUs idle (as here): the
# results meet the GEMV bar, which the GEMM's one fp16 rounding a weight would
# not, and the first 16 tokens equal cq_gemv's 16-token launch bit for bit (the
# same fragments and order).  65 tokens take the GEMM (64 x 32 tiles for the
# 2- and 4-bit fields here: each group's steps in quarters).
@pytest.mark.parametrize("code", [1, 2, 4, 5])
@pytest.mark.parametrize("m", [17, 32, 48, 65])
def test_cq_gemm_few_tokens(code, m, codebooks):
    rng = np.random.default_rng(1700 + code + m)
    rows, cols = 300, 1024
    lv, idx, n16, blob, q, s = oracle_case(rng, rows, cols, code, m, codebooks)
    lay = B.cq_pack_info(rows, cols, 128, code)
    cb = host_codebook(code, codebooks)
    y = host(B.cq_gemm(dev(blob), lay, cb, dev(q), dev(s)))
    if m > 64:
        P.check_cq(y, idx, n16, 128, code, lv, q, s, P.TOL_FOLD, f"cq_gemm code {code} m{m} 300x1024 (GEMM)")
        return
    P.check_cq(y, idx, n16, 128, code, lv, q, s, P.TOL_F32, f"cq_gemm code {code} m{m} 300x1024 (decode kernel)")
    yb = host(B.cq_gemv(dev(blob), lay, cb, dev(q[:16]), dev(s[:16])))
    assert np.array_equal(y[:16], yb)


# The two-half batched kernel on every shape class it meets: K in chunks of
# 16 groups (4096, and 8320 = 65 groups: a ragged last chunk), 2 and 4 row
# blocks a workgroup with ragged ends, and the K split in two workgroups
# added into a zeroed y (16384 columns, one row block a CU); 24 tokens leave
# 8 token columns of the second half empty.
@pytest.mark.parametrize("rows,cols", [(300, 4096), (70, 8320), (5000, 2048), (9000, 512), (40, 16384)])
@pytest.mark.parametrize("m", [24, 32])
def test_cq_gemm_two_token_halves(rows, cols, m, codebooks):
    rng = np.random.default_rng(1800 + rows + cols + m)
    lv, idx, n16, blob, q, s = oracle_case(rng, rows, cols, 4, m, codebooks)
    lay = B.cq_pack_info(rows, cols, 128, 4)
    y = host(B.cq_gemm(dev(blob), lay, host_codebook(4, codebooks), dev(q), dev(s)))
    P.check_cq(y, idx, n16, 128, 4, lv, q, s, P.TOL_F32, f"cq_gemm m{m} {rows}x{cols} (two token halves)")


@pytest.mark.parametrize("rows,cols,batch", [(312, 312, 1), (104, 312, 1), (1092, 312, 1),
                                             (312, 1092, 1), (300, 40, 3), (7, 1000, 16),
                                             (33, 33, 2)])
def test_q4_0_gemv_parity(rows, cols, batch):
    rng = np.random.default_rng(600 + rows + cols + batch)
    w = inputs.weight_matrix(rng, rows, cols)
    x = inputs.activations(rng, batch, cols)
    blk = oq4.encode(w)
    y = host(B.q4_0_gemv(dev(blk.ravel()), rows, cols, dev(x)))
    P.check_q4_0(y, blk, cols, x, label=f"q4_0_gemv {rows}x{cols} b{batch}")


def test_q4_0_stacked_rows_match_separate():
    """Matrices that read the same activations (a layer's q, k, v; gate and
    up), stacked row-wise into one launch, give every row bit for bit the
    result of its own matrix's GEMV launch, and its GEMM result to fp32
    roundoff."""
    rng = np.random.default_rng(1300)
    for group in (((312, 312), (104, 312), (104, 312)), ((1092, 312), (1092, 312)), ((40, 1092), (300, 1092))):
        cols = group[0][1]
        x = dev(inputs.activations(rng, 1, cols))
        blks = [B.q4_0_pack(dev(inputs.weight_matrix(rng, r, cols))) for r, _ in group]
        ys = np.concatenate([host(B.q4_0_gemv(b, r, cols, x)) for b, (r, _) in zip(blks, group)], axis=1)
        yst = host(B.q4_0_gemv(torch.cat(blks), sum(r for r, _ in group), cols, x))
        assert np.array_equal(ys.view(np.uint32), yst.view(np.uint32)), group
        # prefill: the stacked GEMM may take another tile (another order of the
        # fp32 sums), so rows agree to fp32 roundoff
        xm = inputs.activations(rng, 64, cols)
        ym = np.concatenate([host(B.q4_0_gemm(b, r, cols, dev(xm))) for b, (r, _) in zip(blks, group)], axis=1)
        ymst = host(B.q4_0_gemm(torch.cat(blks), sum(r for r, _ in group), cols, dev(xm)))
        mag = np.concatenate([omm.q4_0_magnitude(host(b).reshape(r, -1, 18), cols, xm) for b, (r, _) in zip(blks, group)],
                             axis=1)
        assert np.all(np.abs(ym - ymst) <= 2 * P.TOL_F32 * mag), group


# tall matrices of 9..16 blocks a row take the persistent row-tile kernel
# (16 lanes a row, activations in registers): a full last block ending the
# buffer (512 cols), ragged ones with cols % 4 != 0 (301, 318: 4-byte
# activation loads), and batches split 4+1, 2+1 and 4+2
@pytest.mark.parametrize("rows,cols,batch", [(8192, 512, 1), (9001, 301, 3), (32002, 312, 5),
                                             (8200, 318, 6),
                                             # fewer rows than a 16-row tile, a ragged last tile
                                             (5, 300, 2), (17, 500, 3), (1, 289, 1)])
def test_q4_0_gemv_row_tiles(rows, cols, batch):
    rng = np.random.default_rng(610 + rows + cols + batch)
    w = inputs.weight_matrix(rng, rows, cols)
    x = inputs.activations(rng, batch, cols)
    blk = oq4.encode(w)
    y = host(B.q4_0_gemv(dev(blk.ravel()), rows, cols, dev(x)))
    P.check_q4_0(y, blk, cols, x, label=f"q4_0_gemv rows {rows}x{cols} b{batch}")


# the Minueza layer and head shapes at a prompt's worth of tokens, a ragged
# token count, cols past a whole block (1092) and not a multiple of 4 (33, 101:
# the 4-byte activation loads), single rows, tokens and columns
@pytest.mark.parametrize("rows,cols,m", [(312, 312, 37), (104, 312, 512), (1092, 312, 64),
                                         (312, 1092, 100), (32002, 312, 130), (70, 33, 65),
                                         (129, 101, 3), (1, 1, 1), (5, 64, 1),
                                         # an odd block count with a full last block: that
                                         # block starts 4-byte aligned and ends the buffer
                                         (1, 96, 5), (3, 32, 7), (7, 160, 33)])
def test_q4_0_gemm_parity(rows, cols, m):
    rng = np.random.default_rng(650 + rows + cols + m)
    w = inputs.weight_matrix(rng, rows, cols)
    x = inputs.activations(rng, m, cols)
    blk = oq4.encode(w)
    y = host(B.q4_0_gemm(dev(blk.ravel()), rows, cols, dev(x)))
    P.check_q4_0(y, blk, cols, x, label=f"q4_0_gemm m{m} {rows}x{cols}")
    # every token's row equals the GEMV's sum to fp32 rounding
    g = host(B.q4_0_gemv(dev(blk.ravel()), rows, cols, dev(x[:1])))
    assert np.all(np.abs(y[:1] - g) <= 2 * P.TOL_F32 * omm.q4_0_magnitude(blk, cols, x[:1]))


def test_graph_replays_match_eager(codebooks):
    """Every compute entry point captured in one HIP graph (as the decode and
    prefill benchmarks run them): each of three replays, with eager work and
    synchronisations between them, reproduces the eager results bit for bit."""
    rng = np.random.default_rng(750)
    cb = codebooks[4]
    w = torch.from_numpy(weights(rng, 300, 4096)).to(DEV)
    lay = B.cq_pack_info(300, 4096, 128, 4)
    blob = B.cq_pack(w, lay, cb)
    w3 = torch.from_numpy(weights(rng, 200, 1024)).to(DEV)
    lay3 = B.cq_pack_info(200, 1024, 128, 3)
    blob3 = B.cq_pack(w3, lay3, codebooks[3])
    layt = B.cq_pack_info(200, 1024, 128, ocq.TERNARY_B3)
    blobt = B.cq_pack(w3, layt, None)
    wk = torch.from_numpy(weights(rng, 100, 8192)).to(DEV)
    layk = B.cq_pack_info(100, 8192, 128, 4)
    blobk = B.cq_pack(wk, layk, cb)
    qk, sk = B.act_fwht_quant_a8(dev(inputs.activations(rng, 12, 8192)))
    wq = torch.from_numpy(inputs.weight_matrix(rng, 312, 1092)).to(DEV)
    blk = B.q4_0_pack(wq)
    x1, x4 = (dev(inputs.activations(rng, b, 4096)) for b in (1, 4))
    xp = dev(inputs.activations(rng, 70, 1024))
    xq, xqm = (dev(inputs.activations(rng, b, 1092)) for b in (1, 37))
    f32 = lambda *shape: torch.empty(shape, dtype=torch.float32, device=DEV)
    y1, y4, yp, yq, yqm, yt = f32(1, 300), f32(4, 300), f32(70, 200), f32(1, 312), f32(37, 312), f32(70, 200)
    yk = f32(12, 100)
    qp = torch.empty((70, 1024), dtype=torch.int8, device=DEV)
    sp = f32(70)
    blob_out = torch.empty_like(blob)
    outs = [y1, y4, qp, sp, yp, yq, yqm, blob_out, yt, yk]

    def step():
        B.cq_gemv_f32(blob, lay, cb, x1, y=y1)                 # VALU GEMV, A8 fused
        B.cq_gemv_f32(blob, lay, cb, x4, y=y4)                 # matrix-core GEMV, 4 tokens
        B.act_fwht_quant_a8(xp, q=qp, scale=sp)
        B.cq_gemm(blob3, lay3, codebooks[3], qp, sp, y=yp)
        B.cq_gemm(blobt, layt, None, qp, sp, y=yt)             # base-3 ternary GEMM
        B.cq_gemv(blobk, layk, cb, qk, sk, y=yk)               # K split: zero fill, atomic halves
        B.q4_0_gemv(blk, 312, 1092, xq, y=yq)
        B.q4_0_gemm(blk, 312, 1092, xqm, y=yqm)
        B.cq_pack(w, lay, cb, blob=blob_out)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for t in outs:
            t.zero_()                                        # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (t, r) in enumerate(zip(outs, ref)):
            assert torch.equal(t.view(torch.uint8), r.view(torch.uint8)), f"replay {rep}, output {i}"


# the largest rows each path takes: the int8 GEMV up to 36864 columns (its fp16
# copy of one token fills the 72 KB of LDS; several tokens go one a launch),
# the fused fp32 GEMV up to 16384, the GEMM with a long K
@pytest.mark.parametrize("code", [1, 4])
@pytest.mark.parametrize("entry,rows,cols,batch", [("gemv", 33, 36864, 1), ("gemv", 20, 36864, 3),
                                                   ("f32", 9, 16384, 1), ("f32", 9, 16384, 4),
                                                   ("gemm", 100, 36864, 64)])
def test_maximum_sizes(code, entry, rows, cols, batch, codebooks):
    rng = np.random.default_rng(980 + code + rows + batch)
    lv, idx, n16, blob, q, s = oracle_case(rng, rows, cols, code, batch, codebooks)
    lay = B.cq_pack_info(rows, cols, 128, code)
    cb = host_codebook(code, codebooks)
    if entry == "f32":
        x = inputs.activations(rng, batch, cols)
        q, s = oa8.act_quant_a8(x, 128, "fp32")
        y = host(B.cq_gemv_f32(dev(blob), lay, cb, dev(x)))
    elif entry == "gemv":
        y = host(B.cq_gemv(dev(blob), lay, cb, dev(q), dev(s)))
    else:
        y = host(B.cq_gemm(dev(blob), lay, cb, dev(q), dev(s)))
    tol = P.TOL_FOLD if entry == "gemm" else (P.TOL_F32 if entry == "f32" else P.cq_gemv_tol(cols, batch))
    P.check_cq(y, idx, n16, 128, code, lv, q, s, tol, f"max size {entry} code {code} {rows}x{cols} b{batch}")


# rows wider than the fused launch's 16384 columns: with code buffers,
# cq_gemv_f32 runs the A8 step into them and then cq_gemv (one token and three
# tokens on the VALU GEMV, six on the GEMM kernel)
@pytest.mark.parametrize("rows,cols,batch", [(33, 28672, 1), (20, 36864, 3), (9, 20480, 6)])
def test_cq_gemv_f32_wide_rows(rows, cols, batch, codebooks):
    rng = np.random.default_rng(1700 + rows + batch)
    lv, idx, n16, blob, _, _ = oracle_case(rng, rows, cols, 4, batch, codebooks)
    x = inputs.activations(rng, batch, cols)
    q_ref, s_ref = oa8.act_quant_a8(x, 128, "fp32")
    lay = B.cq_pack_info(rows, cols, 128, 4)
    db = dev(blob)
    q_out = torch.empty((batch, cols), dtype=torch.int8, device=DEV)
    s_out = torch.empty(batch, dtype=torch.float32, device=DEV)
    y = host(B.cq_gemv_f32(db, lay, codebooks[4], dev(x), q_out=q_out, scale_out=s_out))
    assert np.array_equal(host(q_out), q_ref)
    assert np.array_equal(host(s_out).view(np.uint32), s_ref.view(np.uint32))
    y2 = host(B.cq_gemv(db, lay, codebooks[4], q_out, s_out))
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))
    tol = P.TOL_FOLD if batch > 4 else P.cq_gemv_tol(cols, batch)
    P.check_cq(y, idx, n16, 128, 4, lv, q_ref, s_ref, tol, f"cq_gemv_f32 wide rows {rows}x{cols} b{batch}")


def test_results_are_deterministic(codebooks):
    rng = np.random.default_rng(700)
    lv, idx, n16, blob, q, s = oracle_case(rng, 300, 1024, 4, 40, codebooks)
    lay = B.cq_pack_info(300, 1024, 128, 4)
    db, dq, ds = dev(blob), dev(q), dev(s)
    a = host(B.cq_gemv(db, lay, codebooks[4], dq[:4], ds[:4]))
    b = host(B.cq_gemv(db, lay, codebooks[4], dq[:4], ds[:4]))
    c = host(B.cq_gemm(db, lay, codebooks[4], dq, ds))
    d = host(B.cq_gemm(db, lay, codebooks[4], dq, ds))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert np.array_equal(c.view(np.uint32), d.view(np.uint32))
    # the K-split batched GEMV (two halves added into y): the same bits every run
    lv, idx, n16, blob, q, s = oracle_case(rng, 300, 8192, 4, 12, codebooks)
    lay = B.cq_pack_info(300, 8192, 128, 4)
    db, dq, ds = dev(blob), dev(q), dev(s)
    runs = [host(B.cq_gemv(db, lay, codebooks[4], dq, ds)) for _ in range(3)]
    assert all(np.array_equal(r.view(np.uint32), runs[0].view(np.uint32)) for r in runs[1:])


# ------------------------------------------------ full sizes, sampled outputs

def sampled_rows(rng, n, k=48):
    return np.sort(rng.choice(n, size=min(n, k), replace=False))


@pytest.mark.parametrize("rows,cols", inputs.DECODE_8B_SHAPES)
def test_full_size_decode_gemv_sampled(rows, cols, codebooks):
    """8B-class decode shapes: device encode + A8 + GEMV at full size; checked on sampled rows."""
    rng = np.random.default_rng(800 + rows + cols)
    w = inputs.weight_matrix(rng, rows, cols, outliers=True)
    x = inputs.activations(rng, 1, cols)
    lay = B.cq_pack_info(rows, cols, 128, 4)
    blob = B.cq_pack(dev(w), lay, codebooks[4])
    q, s = B.act_fwht_quant_a8(dev(x))
    y = host(B.cq_gemv(blob, lay, codebooks[4], q, s))
    sel = sampled_rows(rng, rows)
    idx, n16 = ocq.encode(w[sel], 128, 4, codebooks[4])
    gi, gn = ocq.split_blob(host(blob), rows, cols, 128, 4)
    assert np.array_equal(gi[sel], idx) and np.array_equal(gn[sel].view(np.uint16), n16.view(np.uint16))
    q_ref, s_ref = oa8.act_quant_a8(x, 128, "fp32")
    assert np.array_equal(host(q), q_ref)
    P.check_cq(y[:, sel], idx, n16, 128, 4, codebooks[4], q_ref, s_ref, P.TOL_F32,
               f"full-size decode {rows}x{cols} (sampled rows)")


# 2..16 tokens on the matrix-core GEMV at full size: one K chunk with 4 and 8
# row blocks per workgroup (14336 and 30000 rows), and K in chunks of 4096
# columns with a partial last chunk and 1, 2 and 4 row blocks per workgroup
@pytest.mark.parametrize("rows,cols,batch,code", [(14336, 4096, 8, 4), (30000, 4096, 5, 1),
                                                  (4096, 14336, 16, 4), (4096, 14336, 3, 3),
                                                  (6000, 4224, 12, 2), (9000, 5120, 16, 4)])
def test_full_size_batched_decode_sampled(rows, cols, batch, code, codebooks):
    rng = np.random.default_rng(850 + rows + cols + batch)
    w = inputs.weight_matrix(rng, rows, cols, outliers=True)
    x = inputs.activations(rng, batch, cols)
    lay = B.cq_pack_info(rows, cols, 128, code)
    cb = host_codebook(code, codebooks)
    blob = B.cq_pack(dev(w), lay, cb)
    q, s = B.act_fwht_quant_a8(dev(x))
    y = host(B.cq_gemv(blob, lay, cb, q, s))
    sel = np.unique(np.concatenate([sampled_rows(rng, rows, 40), np.arange(rows - 3, rows)]))
    idx, n16 = ocq.split_blob(host(blob), rows, cols, 128, code)
    P.check_cq(y[:, sel], idx[sel], n16[sel], 128, code, levels(code, codebooks), host(q), host(s),
               P.cq_gemv_tol(cols, batch), f"full-size batched {rows}x{cols} b{batch} code {code}")


# the prefill shapes (512 tokens, K = 4096), plus shapes that select each
# GEMM tile (128x256 for 14336 / 14200 outputs, 128x128 for 7168 and for the
# ragged 300 x 14000, 64x128 for 4096), with ragged tiles in m and n
@pytest.mark.parametrize("m,rows", [(512, 14336), (512, 4096), (512, 7168), (300, 14000), (512, 14200)])
def test_full_size_prefill_gemm_sampled(m, rows, codebooks):
    rng = np.random.default_rng(900 + rows + m)
    cols = 4096
    w = inputs.weight_matrix(rng, rows, cols)
    x = inputs.activations(rng, m, cols)
    lay = B.cq_pack_info(rows, cols, 128, 4)
    blob = B.cq_pack(dev(w), lay, codebooks[4])
    q, s = B.act_fwht_quant_a8(dev(x))
    y = host(B.cq_gemm(blob, lay, codebooks[4], q, s))
    sel = np.unique(np.concatenate([sampled_rows(rng, rows, 40), np.arange(rows - 3, rows)]))
    idx, n16 = ocq.split_blob(host(blob), rows, cols, 128, 4)
    P.check_cq(y[:, sel], idx[sel], n16[sel], 128, 4, codebooks[4], host(q), host(s), P.TOL_FOLD,
               f"full-size prefill m{m} {rows}x{cols}")


@pytest.mark.parametrize("code", [1, 2, 3, 4, 5])
def test_full_size_bit_sweep_sampled(code, codebooks):
    rng = np.random.default_rng(1000 + code)
    rows, cols = inputs.SWEEP_SHAPE
    w = inputs.weight_matrix(rng, rows, cols, outliers=True)
    lay = B.cq_pack_info(rows, cols, 128, code)
    blob = B.cq_pack(dev(w), lay, host_codebook(code, codebooks))
    sel = sampled_rows(rng, rows, 32)
    lv = levels(code, codebooks)
    idx, n16 = ocq.split_blob(host(blob), rows, cols, 128, code)
    ridx, rn16 = ocq.encode(w[sel], 128, code, lv)
    assert np.array_equal(idx[sel], ridx) and np.array_equal(n16[sel].view(np.uint16), rn16.view(np.uint16))
    for batch in inputs.SWEEP_BATCHES:
        x = inputs.activations(rng, batch, cols)
        q, s = B.act_fwht_quant_a8(dev(x))
        y = host(B.cq_gemv(blob, lay, host_codebook(code, codebooks), q, s))
        P.check_cq(y[:, sel], idx[sel], n16[sel], 128, code, lv, host(q), host(s),
                   P.cq_gemv_tol(cols, batch), f"full-size sweep code {code} b{batch}")


# several tokens: one pass on the int8 matrix cores (K in chunks past 32
# groups, row counts off the 16-row blocks, 16 tokens, one group a row)
@pytest.mark.parametrize("rows,cols,batch", [(300, 512, 2), (130, 4096, 4), (77, 8192, 3), (33, 1024, 16),
                                             (9, 640, 5), (1000, 384, 7), (40, 12288, 6), (64, 16384, 16),
                                             (17, 128, 9), (2000, 4224, 11)])
def test_cq_gemv_ternary_b3_batched(rows, cols, batch, codebooks):
    rng = np.random.default_rng(490 + rows + cols + batch)
    lv, idx, n16, blob, q, s = oracle_case(rng, rows, cols, ocq.TERNARY_B3, batch, codebooks)
    lay = B.cq_pack_info(rows, cols, 128, ocq.TERNARY_B3)
    y = host(B.cq_gemv(dev(blob), lay, None, dev(q), dev(s)))
    P.check_cq(y, idx, n16, 128, ocq.TERNARY_B3, lv, q, s, P.TOL_F32, f"cq_gemv base-3 {rows}x{cols} b{batch}")
    # each token agrees with the one-token product on its own (the same exact
    # group sums; the fp32 sum over groups runs in another order)
    mag = omm.cq_magnitude(idx, n16, 128, ocq.TERNARY_B3, lv, q, s)
    for b in (0, batch - 1):
        y1 = host(B.cq_gemv(dev(blob), lay, None, dev(q[b:b + 1]), dev(s[b:b + 1])))
        assert np.all(np.abs(y1[0] - y[b]) <= 2 * P.TOL_F32 * mag[b]), b
    x = inputs.activations(rng, batch, cols)
    q_out = torch.empty((batch, cols), dtype=torch.int8, device=DEV)
    s_out = torch.empty((batch,), dtype=torch.float32, device=DEV)
    yf = host(B.cq_gemv_f32(dev(blob), lay, None, dev(x), q_out=q_out, scale_out=s_out))
    y2 = host(B.cq_gemv(dev(blob), lay, None, q_out, s_out))
    assert np.array_equal(yf.view(np.uint32), y2.view(np.uint32))


# base-3 prefill: up to 16 tokens the batched decode launch (bit for bit
# cq_gemv's), more tokens (or more than 16384 columns) the base-3 GEMM, here
# in its 64 x 128 tile: ragged token and row tiles, odd group counts, one
# group, a single token past 16384 columns
@pytest.mark.parametrize("rows,cols,m", [(300, 512, 37), (129, 4096, 100), (64, 16384, 17), (1000, 384, 16),
                                         (33, 1024, 1), (257, 1152, 129), (130, 128, 300), (40, 20480, 20),
                                         (31, 16512, 1), (500, 2944, 65)])
def test_cq_gemm_ternary_b3(rows, cols, m, codebooks):
    rng = np.random.default_rng(495 + rows + cols + m)
    lv, idx, n16, blob, q, s = oracle_case(rng, rows, cols, ocq.TERNARY_B3, m, codebooks)
    lay = B.cq_pack_info(rows, cols, 128, ocq.TERNARY_B3)
    y = host(B.cq_gemm(dev(blob), lay, None, dev(q), dev(s)))
    P.check_cq(y, idx, n16, 128, ocq.TERNARY_B3, lv, q, s, P.TOL_F32, f"cq_gemm base-3 m{m} {rows}x{cols}")
    if m <= 16 and cols <= 16384:
        # the same launch as cq_gemv: equal bit for bit
        y16 = host(B.cq_gemv(dev(blob), lay, None, dev(q), dev(s)))
        assert np.array_equal(y16.view(np.uint32), y.view(np.uint32))


# the base-3 GEMM's 128 x 256 (m 512, 14336 rows: the bench's prefill line),
# 128 x 128 and 64 x 128 tiles at full size, ragged in tokens and rows:
# sampled rows against the oracle
@pytest.mark.parametrize("m,rows,cols", [(512, 14336, 4096), (256, 14336, 1024), (300, 14000, 2048),
                                         (512, 4096, 14336)])
def test_full_size_ternary_b3_prefill_sampled(m, rows, cols):
    rng = np.random.default_rng(1200 + rows + m + cols)
    code = ocq.TERNARY_B3
    w = inputs.weight_matrix(rng, rows, cols, outliers=True)
    x = inputs.activations(rng, m, cols)
    lay = B.cq_pack_info(rows, cols, 128, code)
    blob = B.cq_pack(dev(w), lay, None)
    q, s = B.act_fwht_quant_a8(dev(x))
    y = host(B.cq_gemm(blob, lay, None, q, s))
    sel = np.unique(np.concatenate([sampled_rows(rng, rows, 40), np.arange(rows - 3, rows)]))
    idx, n16 = ocq.split_blob(host(blob), rows, cols, 128, code)
    P.check_cq(y[:, sel], idx[sel], n16[sel], 128, code, levels(code, None), host(q), host(s), P.TOL_F32,
               f"full-size base-3 prefill m{m} {rows}x{cols}")


@pytest.mark.parametrize("rows,cols,batch", [(14336, 4096, 16), (4096, 14336, 16), (14336, 4096, 4)])
def test_full_size_ternary_b3_batched_sampled(rows, cols, batch):
    """Base-3 ternary at the sweep shapes, several tokens on the matrix
    cores, in the launch the bench times: sampled rows against the oracle."""
    rng = np.random.default_rng(1150 + rows + batch)
    w = inputs.weight_matrix(rng, rows, cols, outliers=True)
    code = ocq.TERNARY_B3
    lay = B.cq_pack_info(rows, cols, 128, code)
    blob = B.cq_pack(dev(w), lay, None)
    sel = sampled_rows(rng, rows, 32)
    lv = levels(code, None)
    idx, n16 = ocq.split_blob(host(blob), rows, cols, 128, code)
    x = inputs.activations(rng, batch, cols)
    q, s = B.act_fwht_quant_a8(dev(x))
    y = host(B.cq_gemv(blob, lay, None, q, s))
    P.check_cq(y[:, sel], idx[sel], n16[sel], 128, code, lv, host(q), host(s), P.TOL_F32,
               f"full-size base-3 {rows}x{cols} b{batch}")


@pytest.mark.parametrize("rows,cols", [(14336, 4096), (4096, 14336)])
def test_full_size_ternary_b3_sampled(rows, cols):
    """Base-3 ternary at the sweep and down-projection shapes, one token, in
    the launch the bench times: packed on the device (bit-exact on sampled
    rows), product on sampled rows against the oracle."""
    rng = np.random.default_rng(1100 + rows)
    w = inputs.weight_matrix(rng, rows, cols, outliers=True)
    code = ocq.TERNARY_B3
    lay = B.cq_pack_info(rows, cols, 128, code)
    blob = B.cq_pack(dev(w), lay, None)
    sel = sampled_rows(rng, rows, 32)
    lv = levels(code, None)
    idx, n16 = ocq.split_blob(host(blob), rows, cols, 128, code)
    ridx, rn16 = ocq.encode(w[sel], 128, code, lv)
    assert np.array_equal(idx[sel], ridx) and np.array_equal(n16[sel].view(np.uint16), rn16.view(np.uint16))
    x = inputs.activations(rng, 1, cols)
    q, s = B.act_fwht_quant_a8(dev(x))
    y = host(B.cq_gemv(blob, lay, None, q, s))
    P.check_cq(y[:, sel], idx[sel], n16[sel], 128, code, lv, host(q), host(s), P.TOL_F32,
               f"full-size base-3 {rows}x{cols}")


def test_full_size_minueza_pass():
    wl = inputs.minueza_q4_0_pass(layers=2)
    rng = np.random.default_rng(1100)
    for (label, w), x in zip(wl.weights, wl.acts):
        rows, cols = w.shape
        blocks = B.q4_0_pack(dev(w))
        y = host(B.q4_0_gemv(blocks, rows, cols, dev(x)))
        sel = sampled_rows(rng, rows, 32)
        ref_blk = oq4.encode(w[sel])
        got_blk = host(blocks).reshape(rows, -1, 18)
        assert np.array_equal(got_blk[sel], ref_blk), label
        P.check_q4_0(y[:, sel], ref_blk, cols, x, label=f"minueza {label} (sampled rows)")


# ------------------------------------------- mixed-scale rows on every route

def mixed_case(rng, rows, cols, code, batch, codebooks):
    w = inputs.weight_matrix_mixed(rng, rows, cols)
    x = inputs.activations(rng, batch, cols)
    lv = levels(code, codebooks)
    idx, n16 = ocq.encode(w, 128, code, lv)
    return x, lv, idx, n16, ocq.make_blob(idx, n16, 128, code)


# (entry, rows, cols, batch): cq_gemv on the VALU GEMV (1 token; 2 past 4096
# columns; 3 past 16384), on the matrix cores (2 and 9 tokens, one K chunk and
# several) and on the GEMM kernel (6 tokens past 16384 columns); cq_gemv_f32
# fused (1 and 4 tokens) and with code buffers (4 tokens: the matrix cores);
# cq_gemm with norms a group at a time (1152 columns) and 8 to a load (2048)
MIXED_ROUTES = [("gemv", 60, 1024, 1), ("gemv", 60, 1024, 2), ("gemv", 60, 5120, 2),
                ("gemv", 60, 5120, 9), ("gemv", 40, 20480, 6), ("gemv", 40, 20480, 3),
                ("f32", 60, 1024, 1), ("f32", 60, 4096, 4), ("f32_codes", 60, 4096, 4),
                ("gemm", 60, 1152, 37), ("gemm", 300, 2048, 70)]


@pytest.mark.parametrize("code", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("entry,rows,cols,batch", MIXED_ROUTES)
def test_mixed_scale_rows_every_route(entry, rows, cols, batch, code, codebooks):
    """Rows at 1e-3, 1e-4 and 1e-6 of the others (group norms down to fp16
    subnormals), a row of alternately scaled groups and an all-zero row: every
    element within its path's bound of the oracle, the zero row exactly 0."""
    rng = np.random.default_rng(1200 + code * 31 + rows + cols + batch)
    x, lv, idx, n16, blob = mixed_case(rng, rows, cols, code, batch, codebooks)
    lay = B.cq_pack_info(rows, cols, 128, code)
    cb = host_codebook(code, codebooks)
    q, s = oa8.act_quant_a8(x, 128, "fp32")
    if entry == "gemv":
        y = host(B.cq_gemv(dev(blob), lay, cb, dev(q), dev(s)))
        tol = P.cq_gemv_tol(cols, batch)
    elif entry == "gemm":
        y = host(B.cq_gemm(dev(blob), lay, cb, dev(q), dev(s)))
        tol = P.TOL_FOLD
    else:
        codes = entry == "f32_codes"
        q_out = torch.empty((batch, cols), dtype=torch.int8, device=DEV) if codes else None
        s_out = torch.empty((batch,), dtype=torch.float32, device=DEV) if codes else None
        y = host(B.cq_gemv_f32(dev(blob), lay, cb, dev(x), q_out=q_out, scale_out=s_out))
        tol = P.cq_gemv_tol(cols, batch) if codes else P.TOL_F32
    assert np.all(y[:, rows // 2] == 0.0)
    P.check_cq(y, idx, n16, 128, code, lv, q, s, tol, f"mixed {entry} code {code} {rows}x{cols} b{batch}")


@pytest.mark.parametrize("rows,cols,batch", [(60, 1024, 1), (60, 4096, 3), (33, 16384, 1), (40, 8192, 5)])
def test_mixed_scale_rows_base3(rows, cols, batch, codebooks):
    rng = np.random.default_rng(1300 + rows + cols + batch)
    x, lv, idx, n16, blob = mixed_case(rng, rows, cols, ocq.TERNARY_B3, batch, codebooks)
    lay = B.cq_pack_info(rows, cols, 128, ocq.TERNARY_B3)
    q, s = oa8.act_quant_a8(x, 128, "fp32")
    y = host(B.cq_gemv(dev(blob), lay, None, dev(q), dev(s)))
    assert np.all(y[:, rows // 2] == 0.0)
    P.check_cq(y, idx, n16, 128, ocq.TERNARY_B3, lv, q, s, P.TOL_F32, f"mixed base-3 {rows}x{cols} b{batch}")


@pytest.mark.parametrize("entry,rows,cols,m", [("gemv", 60, 312, 1), ("gemv", 60, 1092, 3),
                                               ("gemm", 60, 312, 37), ("gemm", 300, 1092, 100)])
def test_mixed_scale_rows_q4_0(entry, rows, cols, m):
    rng = np.random.default_rng(1400 + rows + cols + m)
    w = inputs.weight_matrix_mixed(rng, rows, cols, group=32)
    x = inputs.activations(rng, m, cols)
    blk = oq4.encode(w)
    fn = B.q4_0_gemv if entry == "gemv" else B.q4_0_gemm
    y = host(fn(dev(blk.ravel()), rows, cols, dev(x)))
    assert np.all(y[:, rows // 2] == 0.0)
    P.check_q4_0(y, blk, cols, x, label=f"mixed q4_0_{entry} {rows}x{cols} m{m}")


def test_gemm_tiny_norm_rows_stay_within_bound(codebooks):
    """A whole matrix of rows scaled by 1e-4 (group norms ~2e-5, fp16
    subnormals) beside normal rows: the GEMM's per-row fold keeps each row's
    error at 2^-11 of its own magnitude."""
    rng = np.random.default_rng(1500)
    rows, cols, m = 256, 4096, 64
    w = inputs.weight_matrix(rng, rows, cols)
    w[::2] *= np.float32(1e-4)
    x = inputs.activations(rng, m, cols)
    lv = codebooks[4]
    idx, n16 = ocq.encode(w, 128, 4, lv)
    q, s = oa8.act_quant_a8(x, 128, "fp32")
    lay = B.cq_pack_info(rows, cols, 128, 4)
    y = host(B.cq_gemm(dev(ocq.make_blob(idx, n16, 128, 4)), lay, lv, dev(q), dev(s)))
    st = P.check_cq(y, idx, n16, 128, 4, lv, q, s, P.TOL_FOLD, "gemm tiny-norm rows")
    assert st["worst_row_rel"] < 2e-3


# ---------------------------------------------- the lookup-table GEMV (T-MAC)

# 1..4 tokens in one launch (4 side by side, 3 with a zero fourth), 5 and 16
# in several; widths up to its 8192 limit, where the ternary tables of two
# tokens no longer fit and the launches take fewer; rows shorter than a wave
# of chunks (128, 384) and several chunks a lane (8192)
@pytest.mark.parametrize("code", [1, 5])
@pytest.mark.parametrize("rows,cols,batch", [(300, 512, 1), (130, 4096, 1), (130, 4096, 2), (77, 4096, 3),
                                             (64, 4096, 4), (33, 8192, 1), (33, 8192, 4), (5, 128, 2),
                                             (1000, 384, 5), (1, 256, 1), (40, 1024, 16)])
def test_cq_gemv_lut_parity(code, rows, cols, batch, codebooks):
    rng = np.random.default_rng(1700 + code * 3 + rows + cols + batch)
    lv, idx, n16, blob, q, s = oracle_case(rng, rows, cols, code, batch, codebooks)
    lay = B.cq_pack_info(rows, cols, 128, code)
    y = host(B.cq_gemv_lut(dev(blob), lay, dev(q), dev(s)))
    P.check_cq(y, idx, n16, 128, code, lv, q, s, P.TOL_F32, f"cq_gemv_lut code {code} {rows}x{cols} b{batch}")


@pytest.mark.parametrize("code", [1, 5])
def test_cq_gemv_lut_mixed_scale_rows(code, codebooks):
    rng = np.random.default_rng(1750 + code)
    x, lv, idx, n16, blob = mixed_case(rng, 60, 4096, code, 3, codebooks)
    q, s = oa8.act_quant_a8(x, 128, "fp32")
    y = host(B.cq_gemv_lut(dev(blob), B.cq_pack_info(60, 4096, 128, code), dev(q), dev(s)))
    assert np.all(y[:, 30] == 0.0)
    P.check_cq(y, idx, n16, 128, code, lv, q, s, P.TOL_F32, f"mixed cq_gemv_lut code {code}")
