"""Lloyd-Max codebooks (oracle; test infrastructure only).

Needle .cact/W4A8 article, section 1: the 2-, 3- and 4-bit codebooks (4, 8
and 16 levels) are fit offline by Lloyd-Max on 400,000 Gaussian samples for
200 iterations, and stored back to back in the file header, indexed by bit
width at run time.  The mmap article adds two codebook-free sets whose levels
are analytic and built into the engine: ternary (bits code 5), {-c, 0, +c},
and binary (bits code 1), {-sqrt(2/pi), +sqrt(2/pi)}.

Readings taken where the pages are silent:

* Levels live on the N(0,1) scale (sqrt(2/pi) is the two-level Lloyd-Max
  optimum for N(0,1)).
* Fit procedure: fold the samples to |z|, fit L/2 positive levels and mirror
  them, so the table is exactly symmetric.  Levels start at the empirical
  quantiles p_i = (i + 1/2)/(L/2) of |z|: with the sorted values x_(0..n-1),
  h = (n-1)*p_i, j = floor(h), level = x_(j) + (h-j)*(x_(j+1) - x_(j)).
  Each iteration puts the cell boundaries at the midpoints of adjacent levels
  (the first cell starts at 0; a sample on a boundary goes to the upper cell)
  and moves every level to the mean of its cell; an empty cell keeps its level.
* Summation order of a cell's sum (fixed so that a device fit can match it
  bit for bit): the samples, in their given order, are cut into blocks of
  512; each block is summed left to right, then the block sums are added
  left to right.
* The table shipped to the kernels is each fitted level rounded (half-even)
  to the nearest bfloat16-representable value, held as fp32.
* Ternary c is the three-level Lloyd-Max optimum for N(0,1): the fixed point
  of c = E[|Z| : |Z| >= c/2].
"""
from __future__ import annotations

import math

import numpy as np

from .fp import bf16_rne

SAMPLE_COUNT = 400_000
ITERATIONS = 200
SUM_BLOCK = 512
CODEBOOK_LEVELS = {2: 4, 3: 8, 4: 16}      # bits -> number of levels


def ordered_sum(v: np.ndarray, block: int = SUM_BLOCK) -> float:
    """Sum in the fixed order: blocks of ``block`` left to right, then blocks."""
    v = np.asarray(v, dtype=np.float64)
    nb = -(-v.size // block)
    padded = np.zeros(nb * block)
    padded[: v.size] = v                       # adding +0.0 changes no sum
    partial = np.cumsum(padded.reshape(nb, block), axis=1)[:, -1]
    return float(np.cumsum(partial)[-1])


def quantile_init(a_sorted: np.ndarray, half: int) -> np.ndarray:
    """Empirical quantiles (i + 1/2)/half by linear interpolation of order stats."""
    n = a_sorted.size
    p = (np.arange(half, dtype=np.float64) + 0.5) / half
    h = (n - 1) * p
    j = np.floor(h).astype(np.int64)
    t = h - j
    j1 = np.minimum(j + 1, n - 1)
    return a_sorted[j] + t * (a_sorted[j1] - a_sorted[j])


def lloyd_max_fit(samples: np.ndarray, levels: int, iters: int = ITERATIONS) -> np.ndarray:
    """Sample-based Lloyd-Max fit, returned ascending in fp64 (unrounded)."""
    if levels < 2 or levels % 2:
        raise ValueError("sample fit takes an even number of levels")
    a = np.abs(np.asarray(samples, dtype=np.float64))
    half = levels // 2
    pos = quantile_init(np.sort(a), half)
    nb = -(-a.size // SUM_BLOCK)
    members = np.zeros((half, nb * SUM_BLOCK))   # row c holds a where cell == c, else +0.0
    cols = np.arange(a.size)
    for _ in range(iters):
        bounds = 0.5 * (pos[:-1] + pos[1:])
        cell = np.searchsorted(bounds, a, side="right")
        counts = np.bincount(cell, minlength=half)
        members.fill(0.0)
        members[cell, cols] = a
        # same order as ordered_sum(): each block left to right, then the blocks
        partial = np.cumsum(members.reshape(half, nb, SUM_BLOCK), axis=2)[:, :, -1]
        sums = np.cumsum(partial, axis=1)[:, -1]
        pos = np.where(counts > 0, sums / np.maximum(counts, 1), pos)
    return np.concatenate([-pos[::-1], pos])


def _phi(x: float) -> float:
    return math.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)


def _tail(x: float) -> float:
    """P(Z >= x) for Z ~ N(0,1)."""
    return 0.5 * math.erfc(x / math.sqrt(2.0))


def half_normal_centroid(lo: float, hi: float) -> float:
    """E[Z : lo <= Z < hi] for Z ~ N(0,1), 0 <= lo < hi <= inf."""
    num = _phi(lo) - (0.0 if math.isinf(hi) else _phi(hi))
    den = _tail(lo) - (0.0 if math.isinf(hi) else _tail(hi))
    return num / den


def lloyd_max_quadrature(levels: int, tol: float = 1e-15, max_iter: int = 100_000) -> np.ndarray:
    """Lloyd-Max levels for the exact N(0,1) density (pin only), ascending.

    Same iteration as the sample fit, with every cell mean taken from the
    closed form of the truncated normal and iterated to a fixed point.
    Odd ``levels`` put one level at 0 (its cell is symmetric about 0).
    """
    half = levels // 2
    odd = levels % 2
    pos = np.array([_quantile_half_normal((i + 0.5 + 0.5 * odd) / (half + 0.5 * odd))
                    for i in range(half)])
    for _ in range(max_iter):
        if odd:
            bounds = [0.5 * pos[0]] + [0.5 * (pos[i] + pos[i + 1]) for i in range(half - 1)]
        else:
            bounds = [0.0] + [0.5 * (pos[i] + pos[i + 1]) for i in range(half - 1)]
        bounds.append(math.inf)
        new = np.array([half_normal_centroid(bounds[i], bounds[i + 1]) for i in range(half)])
        done = np.max(np.abs(new - pos)) <= tol
        pos = new
        if done:
            break
    mid = [0.0] if odd else []
    return np.concatenate([-pos[::-1], mid, pos])


def _quantile_half_normal(p: float) -> float:
    """Inverse CDF of |Z| by bisection (only used to seed the quadrature fit)."""
    lo, hi = 0.0, 40.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if 1.0 - 2.0 * _tail(mid) < p:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def lloyd_max_mse(levels: np.ndarray) -> float:
    """Mean squared error of nearest-level quantization of N(0,1) (closed form)."""
    lv = np.sort(np.asarray(levels, dtype=np.float64))
    bounds = [-math.inf] + [0.5 * (lv[i] + lv[i + 1]) for i in range(len(lv) - 1)] + [math.inf]
    mse = 0.0
    for i, c in enumerate(lv):
        a, b = bounds[i], bounds[i + 1]
        # E[(Z-c)^2 1{a<=Z<b}] = E[Z^2 1] - 2c E[Z 1] + c^2 P
        p = _cdf(b) - _cdf(a)
        m1 = _phi(a) - _phi(b)
        m2 = p + (a * _phi(a) if math.isfinite(a) else 0.0) - (b * _phi(b) if math.isfinite(b) else 0.0)
        mse += m2 - 2.0 * c * m1 + c * c * p
    return mse


def _cdf(x: float) -> float:
    if math.isinf(x):
        return 1.0 if x > 0 else 0.0
    return 0.5 * math.erfc(-x / math.sqrt(2.0))


def ternary_c() -> float:
    """Three-level Lloyd-Max optimum c for N(0,1): c = E[Z : Z >= c/2]."""
    c = 1.0
    for _ in range(10_000):
        nxt = half_normal_centroid(0.5 * c, math.inf)
        if nxt == c:
            break
        c = nxt
    return c


def binary_level() -> float:
    """Two-level optimum for N(0,1): E|Z| = sqrt(2/pi)."""
    return math.sqrt(2.0 / math.pi)


def shipped_table(raw_levels: np.ndarray) -> np.ndarray:
    """Round each fitted level to bfloat16 precision (half-even), as fp32."""
    return np.array([bf16_rne(float(v)) for v in raw_levels], dtype=np.float32)


def fit_codebooks(samples: np.ndarray, iters: int = ITERATIONS) -> dict:
    """cb2, cb3, cb4 shipped tables keyed by bits."""
    return {b: shipped_table(lloyd_max_fit(samples, n, iters)) for b, n in CODEBOOK_LEVELS.items()}


def analytic_levels(code: int) -> np.ndarray:
    """fp32 levels of the built-in sets: code 1 binary, code 5 ternary."""
    if code == 1:
        c = binary_level()
        return np.array([-c, c], dtype=np.float32)
    if code == 5:
        c = ternary_c()
        return np.array([-c, 0.0, c], dtype=np.float32)
    raise ValueError("analytic sets are bits codes 1 and 5")
