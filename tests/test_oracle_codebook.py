"""Pins for the oracle's Lloyd-Max codebooks and analytic sets (CPU)."""
from __future__ import annotations

import math

import numpy as np
import pytest
from scipy import integrate, stats

from oracle import codebook as cb
from tests.conftest import read_golden_rows


def golden_levels():
    out = {}
    for lv, pos, mse in read_golden_rows("lloyd_max_gaussian.txt"):
        out[int(lv)] = (np.array([float(v) for v in pos.split()]), float(mse))
    return out


def scipy_centroid(a, b):
    """E[Z : a <= Z < b] for N(0,1) by numerical integration (library pin)."""
    num = integrate.quad(lambda z: z * stats.norm.pdf(z), a, b, epsabs=1e-14, epsrel=1e-13)[0]
    den = stats.norm.cdf(b) - stats.norm.cdf(a)
    return num / den


@pytest.mark.parametrize("levels", [2, 3, 4, 8, 16])
def test_quadrature_fit_matches_textbook_and_scipy(levels):
    lv = cb.lloyd_max_quadrature(levels)
    pos_ref, mse_ref = golden_levels()[levels]
    assert np.all(np.diff(lv) > 0)
    assert np.array_equal(lv, -lv[::-1])
    assert np.max(np.abs(lv[lv >= 0] - pos_ref)) < 2e-4
    assert abs(cb.lloyd_max_mse(lv) - mse_ref) < 1e-3 * mse_ref
    # centroid condition checked with scipy's integrator, cell by cell
    bounds = [-math.inf] + list(0.5 * (lv[1:] + lv[:-1])) + [math.inf]
    for i, c in enumerate(lv):
        assert abs(scipy_centroid(bounds[i], bounds[i + 1]) - c) < 1e-10
    # closed-form MSE against numerical integration
    mse_num = sum(integrate.quad(lambda z, c=c: (z - c) ** 2 * stats.norm.pdf(z), bounds[i], bounds[i + 1],
                                 epsabs=1e-14)[0] for i, c in enumerate(lv))
    assert abs(mse_num - cb.lloyd_max_mse(lv)) < 1e-10


def test_binary_level_is_the_pages_sqrt_2_over_pi():
    # the mmap article prints the binary set as +-sqrt(2/pi)
    assert cb.binary_level() == math.sqrt(2.0 / math.pi)
    assert abs(cb.lloyd_max_quadrature(2)[1] - math.sqrt(2.0 / math.pi)) < 1e-14
    lv = cb.analytic_levels(1)
    assert lv.dtype == np.float32 and lv[1] == np.float32(math.sqrt(2.0 / math.pi)) and lv[0] == -lv[1]


def test_ternary_c_is_three_level_optimum():
    c = cb.ternary_c()
    assert abs(scipy_centroid(c / 2, math.inf) - c) < 1e-12
    assert abs(c - cb.lloyd_max_quadrature(3)[2]) < 1e-12
    # MSE of {-c,0,c} is a strict local minimum in c
    f = lambda cc: cb.lloyd_max_mse(np.array([-cc, 0.0, cc]))
    assert f(c) < f(c * 1.01) and f(c) < f(c * 0.99)
    lv = cb.analytic_levels(5)
    assert lv[1] == 0.0 and lv[2] == np.float32(c) and lv[0] == -lv[2]


@pytest.mark.slow
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_sample_fit_invariants(gaussian400k, raw_fits, bits):
    levels = cb.CODEBOOK_LEVELS[bits]
    raw = raw_fits[bits]
    assert np.array_equal(raw, -raw[::-1])          # exact symmetry
    assert np.all(np.diff(raw) > 0)                 # strictly increasing
    # centroid condition on the samples themselves (after 200 iterations)
    a = np.abs(gaussian400k)
    pos = raw[raw > 0]
    bounds = np.concatenate([[0.0], 0.5 * (pos[1:] + pos[:-1]), [np.inf]])
    for i, c in enumerate(pos):
        sel = a[(a >= bounds[i]) & (a < bounds[i + 1])]
        assert abs(sel.mean() - c) < 1e-3
    # within sampling error of the exact N(0,1) optimum
    assert np.max(np.abs(raw - cb.lloyd_max_quadrature(levels))) < 3e-2


def test_sample_fit_two_levels_is_mean_abs(gaussian400k):
    raw = cb.lloyd_max_fit(gaussian400k, 2, iters=1)
    assert abs(raw[1] - np.mean(np.abs(gaussian400k))) < 1e-12


@pytest.mark.slow
def test_shipped_tables_are_bf16_and_close(codebooks, raw_fits):
    for bits, table in codebooks.items():
        assert table.dtype == np.float32
        assert table.shape == (cb.CODEBOOK_LEVELS[bits],)
        low16 = table.view(np.uint32) & 0xFFFF
        assert np.all(low16 == 0)                   # bf16-representable
        raw = raw_fits[bits]
        assert np.all(np.abs(table - raw) <= 2.0 ** -8 * np.abs(raw))   # unit roundoff of an 8-bit significand
        assert np.array_equal(table, -table[::-1])


def test_fixed_summation_order_matches_scalar_definition(gaussian400k):
    """The vectorized fit adds in the documented order (blocks of 512, then blocks)."""
    z = gaussian400k[:5000]
    a = np.abs(z)
    half = 4
    pos = cb.quantile_init(np.sort(a), half)
    for _ in range(3):
        bounds = 0.5 * (pos[:-1] + pos[1:])
        cell = np.searchsorted(bounds, a, side="right")
        cnt = np.bincount(cell, minlength=half)
        sums = []                                   # scalar loops in the stated order
        for c in range(half):
            tot = 0.0
            for b0 in range(0, a.size, cb.SUM_BLOCK):
                part = 0.0
                for i in range(b0, min(b0 + cb.SUM_BLOCK, a.size)):
                    if cell[i] == c:
                        part += float(a[i])
                tot += part
            sums.append(tot)
        pos = np.where(cnt > 0, np.array(sums) / np.maximum(cnt, 1), pos)
    assert np.array_equal(cb.lloyd_max_fit(z, 8, iters=3)[half:], pos)


def test_quantile_init_is_interpolated_order_statistic():
    a = np.sort(np.array([0.5, 0.1, 0.9, 0.3, 0.7]))
    # n = 5, p = 0.25 and 0.75 -> h = 1.0 and 3.0: exact order statistics
    assert np.array_equal(cb.quantile_init(a, 2), np.array([0.3, 0.7]))
    # numpy's default 'linear' quantile agrees away from its lerp special case
    r = np.random.default_rng(0).random(1001)
    assert np.allclose(cb.quantile_init(np.sort(r), 8), np.quantile(r, (np.arange(8) + 0.5) / 8), rtol=0, atol=1e-15)
