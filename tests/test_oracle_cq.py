"""Pins for the oracle's CQ encode / pack / decode (CPU)."""
from __future__ import annotations

import itertools
import math

import numpy as np
import pytest

from oracle import codebook as cb
from oracle import cq
from oracle.fp import fp16_rne
from tests.conftest import read_golden_rows
from tests.test_oracle_hadamard_fp import parity_hadamard


def toy_levels(code):
    """Level tables for the brute-force cases: the analytic sets, and the exact
    N(0,1) Lloyd-Max levels (quadrature fit) rounded to bf16 for codes 2-4."""
    if code in (cq.BINARY, cq.TERNARY):
        return cb.analytic_levels(code)
    return cb.shipped_table(cb.lloyd_max_quadrature(cq.NUM_LEVELS[code]))


def test_packing_matches_hand_built_bytes():
    for bits, idx, expect in read_golden_rows("packing_bytes.txt"):
        b = int(bits)
        ids = np.array([[int(v) for v in idx.split()]], dtype=np.uint8)
        want = np.array([int(v, 16) for v in expect.split()], dtype=np.uint8)
        got = cq.pack_indices(ids, b)
        assert np.array_equal(got[0], want), (bits, idx)
        assert np.array_equal(cq.unpack_indices(got, ids.shape[1], b), ids)


def test_pack_trits_golden():
    """Base-3 bytes worked by hand from the packing rule (tests/golden/packing_trits.txt)."""
    patterns = {"mod3": np.arange(128) % 3, "two": np.full(128, 2), "zero": np.zeros(128, int),
                "one": np.ones(128, int)}
    for name, j, value in read_golden_rows("packing_trits.txt"):
        ids = np.tile(patterns[name], 2).reshape(1, 256).astype(np.uint8)   # two groups
        got = cq.pack_trits(ids, 128)
        assert got.shape == (1, 52)
        assert got[0, int(j)] == int(value), (name, j)
        assert got[0, 26 + int(j)] == int(value), (name, j)       # the second group's byte j
        assert np.array_equal(cq.unpack_trits(got, 256, 128), ids)


def test_pack_trits_digit_positions():
    """Digit i of byte j is index 5j+i: brute force over every position of a
    small group (G = 8: two bytes, the second with two padding digits)."""
    for p in range(8):
        for v in (0, 2):
            ids = np.ones((1, 8), dtype=np.uint8)
            ids[0, p] = v
            got = cq.pack_trits(ids, 8).astype(int)[0]
            j, i = divmod(p, 5)
            want = [121, 121]                       # all digits 1 (padding too)
            want[j] += (v - 1) * 3 ** i
            assert list(got) == want, (p, v)
    rng = np.random.default_rng(6)
    ids = rng.integers(0, 3, size=(5, 384)).astype(np.uint8)
    packed = cq.pack_trits(ids, 128)
    assert packed.max() <= 242 and packed.shape == (5, 3 * 26)
    assert np.array_equal(cq.unpack_trits(packed, 384, 128), ids)
    with pytest.raises(ValueError):
        cq.unpack_trits(np.full((1, 26), 243, np.uint8), 128, 128)
    with pytest.raises(ValueError):
        cq.pack_trits(np.full((1, 128), 3, np.uint8), 128)


def test_ternary_b3_blob_decodes_like_the_2bit_blob():
    """Codes 5 and 6 share levels and encode; only the packing differs, so the
    two blobs decode to the same weights and the layouts differ only in size."""
    rng = np.random.default_rng(66)
    w = (rng.standard_normal((9, 512)) * 0.02).astype(np.float32)
    lv = cq.levels_for(cq.TERNARY)
    assert np.array_equal(cq.levels_for(cq.TERNARY_B3), lv)
    i5, n5 = cq.encode(w, 128, cq.TERNARY, lv)
    i6, n6 = cq.encode(w, 128, cq.TERNARY_B3, lv)
    assert np.array_equal(i5, i6) and np.array_equal(n5, n6)
    b6 = cq.make_blob(i6, n6, 128, cq.TERNARY_B3)
    ri, rn = cq.split_blob(b6, 9, 512, 128, cq.TERNARY_B3)
    assert np.array_equal(ri, i6) and np.array_equal(rn, n6)
    w5 = cq.decode(i5, n5, 128, cq.TERNARY, lv)
    w6 = cq.decode(ri, rn, 128, cq.TERNARY_B3, lv)
    assert np.array_equal(w5, w6)
    info = cq.pack_info(14336, 4096, 128, cq.TERNARY_B3)
    assert info["idx_row_bytes"] == 32 * 26 and info["index_bits"] == 0 and info["levels"] == 3
    # 26 index bytes + a 2-byte norm per 128 weights: 1.75 bits per weight, against 2.125
    bpw = lambda c: 8 * (cq.pack_info(1, 128, 128, c)["idx_row_bytes"] + 2) / 128
    assert bpw(cq.TERNARY_B3) == 1.75 and bpw(cq.TERNARY) == 2.125


@pytest.mark.parametrize("b", [1, 2, 3, 4])
def test_pack_roundtrip_and_bit_positions(b):
    rng = np.random.default_rng(b)
    ids = rng.integers(0, 1 << b, size=(7, 256)).astype(np.uint8)
    packed = cq.pack_indices(ids, b)
    assert packed.shape == (7, 256 * b // 8)
    assert np.array_equal(cq.unpack_indices(packed, 256, b), ids)
    # independent bit-level check: bit (b*j + t) of the row stream is bit t of idx[j]
    bits = np.unpackbits(packed, axis=1, bitorder="little")
    for j in range(0, 256, 37):
        for t in range(b):
            assert bits[3, b * j + t] == (ids[3, j] >> t) & 1


def test_pack_info_sizes():
    # 4-bit, 14336 x 4096, group 128: 2048 B/row of indices + 32 fp16 norms/row
    info = cq.pack_info(14336, 4096, 128, 4)
    assert info["idx_row_bytes"] == 2048
    assert info["idx_bytes"] + 2 * info["norms_count"] == 30_277_632
    assert info["norms_offset"] % 64 == 0 and info["total_bytes"] % 64 == 0
    sizes = {code: cq.pack_info(14336, 4096, 128, code) for code in (1, 2, 3, 4, 5)}
    payload = {c: s["idx_bytes"] + 2 * s["norms_count"] for c, s in sizes.items()}
    assert payload == {1: 8_257_536, 2: 15_597_568, 3: 22_937_600, 4: 30_277_632, 5: 15_597_568}
    with pytest.raises(ValueError):
        cq.pack_info(4, 100, 128, 4)          # cols not a multiple of group
    with pytest.raises(ValueError):
        cq.pack_info(4, 128, 128, 7)          # unknown bits code
    # base-3 ternary: 14336 x 32 groups x 26 bytes + norms
    b3 = cq.pack_info(14336, 4096, 128, 6)
    assert b3["idx_bytes"] + 2 * b3["norms_count"] == 14336 * 32 * 28 == 12_845_056


@pytest.mark.parametrize("code,g", [(cq.BINARY, 8), (cq.TERNARY, 8), (cq.B2, 8), (cq.B3, 4), (cq.B4, 4)])
def test_encode_is_brute_force_nearest_codeword(code, g):
    """Indices equal the exhaustive argmin over all L^G codewords of ||t - c||^2,
    with t = sqrt(G) * H w / ||H w|| computed from the explicit Hadamard matrix."""
    lv = toy_levels(code).astype(np.float64)
    L = len(lv)
    words = np.array(list(itertools.product(range(L), repeat=g)))      # [L^g, g]
    cw = lv[words]
    hn = parity_hadamard(g) / math.sqrt(g)
    rng = np.random.default_rng(10 + code)
    cols = 8                                      # whole bytes per row for every width
    w = (0.02 * rng.standard_normal((40, cols))).astype(np.float32)
    idx, n16 = cq.encode(w, g, code, toy_levels(code))
    for r in range(w.shape[0]):
        for gi in range(cols // g):
            wg = w[r, gi * g:(gi + 1) * g].astype(np.float64)
            y = hn @ wg
            t = math.sqrt(g) * y / np.linalg.norm(y)
            best = words[np.argmin(np.sum((cw - t) ** 2, axis=1))]
            assert np.array_equal(idx[r, gi * g:(gi + 1) * g], best), (code, r, gi)
            assert float(n16[r, gi]) == fp16_rne(np.linalg.norm(wg))


@pytest.mark.parametrize("code,expect", [(cq.BINARY, 0), (cq.B2, 1), (cq.B3, 3), (cq.B4, 7), (cq.TERNARY, 1)])
def test_zero_group_gets_level_nearest_zero_and_decodes_to_zero(code, expect):
    w = np.zeros((2, 128), dtype=np.float32)
    w[1] = np.linspace(-1, 1, 128, dtype=np.float32)
    lv = toy_levels(code)
    idx, n16 = cq.encode(w, 128, code, lv)
    assert np.all(idx[0] == expect)
    assert n16[0, 0] == 0
    wh = cq.decode(idx, n16, 128, code, lv)
    assert np.all(wh[0] == 0.0)


def test_decode_matches_explicit_formula():
    """w_hat_g = norm/sqrt(G) * H cb[idx_g] with H the explicit normalized matrix."""
    rng = np.random.default_rng(11)
    g = 128
    lv = toy_levels(cq.B4)
    idx = rng.integers(0, 16, size=(3, 2 * g)).astype(np.uint8)
    n16 = (rng.random((3, 2)) + 0.1).astype(np.float16)
    wh = cq.decode(idx, n16, g, cq.B4, lv)
    hn = parity_hadamard(g) / math.sqrt(g)
    for r in range(3):
        for gi in range(2):
            c = lv.astype(np.float64)[idx[r, gi * g:(gi + 1) * g]]
            ref = float(n16[r, gi]) / math.sqrt(g) * (hn @ c)
            assert np.max(np.abs(wh[r, gi * g:(gi + 1) * g] - ref)) < 1e-14


def test_ternary_field_value_three_decodes_to_zero():
    lv = cb.analytic_levels(5)
    idx = np.full((1, 128), 3, dtype=np.uint8)
    wh = cq.decode(idx, np.ones((1, 1), dtype=np.float16), 128, cq.TERNARY, lv)
    assert np.all(wh == 0)


@pytest.mark.slow
def test_cb4_distortion_matches_lloyd_max_mse(codebooks):
    """Statistical pin: relative MSE ~ D_4 and ||w_hat||^2/||w||^2 ~ 1 - D_4."""
    rng = np.random.default_rng(12)
    w = (0.02 * rng.standard_normal((256, 1024))).astype(np.float32)
    lv = codebooks[4]
    idx, n16 = cq.encode(w, 128, 4, lv)
    wh = cq.decode(idx, n16, 128, 4, lv)
    d4 = cb.lloyd_max_mse(cb.lloyd_max_quadrature(16))
    rel = cq.quantization_mse(w, wh)
    assert abs(rel - d4) < 1.5e-3
    # t lies exactly on the sqrt(G)-sphere rather than being i.i.d. N(0,1), so the
    # energy ratio only approximates 1 - D; a scale slip (a lost sqrt(G) or norm)
    # would move it by orders of magnitude.
    energy = np.sum(wh ** 2) / np.sum(w.astype(np.float64) ** 2)
    assert abs(energy - (1 - d4)) < 5e-3


def test_blob_roundtrip_and_layout():
    rng = np.random.default_rng(13)
    for code in (1, 2, 3, 4, 5):
        info = cq.pack_info(5, 256, 128, code)
        idx = rng.integers(0, cq.NUM_LEVELS[code], size=(5, 256)).astype(np.uint8)
        n16 = rng.random((5, 2)).astype(np.float16)
        blob = cq.make_blob(idx, n16, 128, code)
        assert blob.size == info["total_bytes"]
        i2, n2 = cq.split_blob(blob, 5, 256, 128, code)
        assert np.array_equal(i2, idx) and np.array_equal(n2.view(np.uint16), n16.view(np.uint16))
        # norms start at the 64-aligned offset, little-endian fp16
        off = info["norms_offset"]
        assert off % 64 == 0 and off >= info["idx_bytes"]
        assert blob[off] == n16.view(np.uint16)[0, 0] & 0xFF


def test_encode_range_errors():
    w = np.full((1, 128), 1.0e4, dtype=np.float32)     # ||w|| = 1.13e5 > 65504
    with pytest.raises(OverflowError):
        cq.encode(w, 128, 4, toy_levels(4))
    w = np.zeros((1, 128), dtype=np.float32)
    w[0, 3] = np.nan
    with pytest.raises(ValueError):
        cq.encode(w, 128, 4, toy_levels(4))
