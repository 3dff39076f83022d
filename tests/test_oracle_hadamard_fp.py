"""Pins for the oracle's Hadamard transform and exact rounding helpers (CPU)."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from oracle import fp, hadamard


def parity_hadamard(g: int) -> np.ndarray:
    """H_u[i, j] = (-1)^popcount(i & j): a closed form independent of the recursion."""
    i = np.arange(g)[:, None]
    j = np.arange(g)[None, :]
    bits = np.vectorize(lambda v: bin(int(v)).count("1"))(i & j)
    return np.where(bits % 2 == 0, 1, -1).astype(np.int64)


@pytest.mark.parametrize("g", [1, 2, 4, 8, 16, 32, 64, 128])
def test_sylvester_matches_parity_form_and_is_orthogonal(g):
    h = hadamard.sylvester(g)
    assert np.array_equal(h, parity_hadamard(g))
    assert np.array_equal(h @ h, g * np.eye(g, dtype=np.int64))
    assert np.array_equal(h, h.T)
    hn = h / math.sqrt(g)
    assert np.max(np.abs(hn @ hn - np.eye(g))) < 1e-15


@pytest.mark.parametrize("g", [2, 8, 128])
def test_fwht_equals_matrix_product(g):
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 3, g))
    ref = x @ parity_hadamard(g).T.astype(np.float64)
    assert np.max(np.abs(hadamard.fwht_u(x) - ref)) < 1e-12 * g
    # integer inputs: the butterfly is exact
    xi = rng.integers(-1000, 1000, size=(7, g)).astype(np.float64)
    assert np.array_equal(hadamard.fwht_u(xi), xi @ parity_hadamard(g).T)


def test_fwht_unit_vectors_and_norm():
    g = 128
    e0 = np.zeros(g)
    e0[0] = 1.0
    assert np.array_equal(hadamard.fwht_u(e0), np.ones(g))
    rng = np.random.default_rng(2)
    x = rng.standard_normal((10, g))
    assert np.allclose(np.linalg.norm(hadamard.fwht(x), axis=1), np.linalg.norm(x, axis=1), rtol=1e-14)
    # applying the normalized transform twice returns the input
    assert np.max(np.abs(hadamard.fwht(hadamard.fwht(x)) - x)) < 1e-13


def test_fwht_fp32_mode_within_fp32_bound():
    g = 128
    rng = np.random.default_rng(3)
    x = rng.standard_normal((50, g)).astype(np.float32)
    u32 = hadamard.fwht_u(x, dtype=np.float32)
    assert u32.dtype == np.float32
    ref = x.astype(np.float64) @ parity_hadamard(g).T
    # 7 stages, each one rounding of magnitude <= 2^-24 * |partial sum|
    bound = 7 * 2.0 ** -24 * (np.abs(x).astype(np.float64) @ np.ones((g, g)))
    assert np.all(np.abs(u32 - ref) <= bound + 1e-30)
    # small integers stay exact in fp32
    xi = rng.integers(-100, 100, size=(4, g)).astype(np.float32)
    assert np.array_equal(hadamard.fwht_u(xi, dtype=np.float32), (xi.astype(np.int64) @ parity_hadamard(g).T).astype(np.float32))


def test_fwht_rejects_non_power_of_two():
    with pytest.raises(ValueError):
        hadamard.fwht_u(np.zeros(12))


def test_fp16_rne_matches_numpy_on_fp32_inputs():
    rng = np.random.default_rng(4)
    v32 = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(3.0),
        (rng.random(2000).astype(np.float32) * np.float32(6e-5)),     # subnormal range
        np.float32([0.0, 65504.0, 65519.0, 1.0, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26]),
    ])
    lib = v32.astype(np.float16).astype(np.float64)      # numpy: correctly rounded
    mine = np.array([fp.fp16_rne(float(v)) for v in v32])
    assert np.array_equal(lib, mine)


def test_fp16_rne_rounds_once_from_fp64():
    # 1 + 2^-11 is the midpoint between fp16 1.0 and 1 + 2^-10: half-even -> 1.0
    assert fp.fp16_rne(1.0 + 2.0 ** -11) == 1.0
    # just above the midpoint: must go up.  Via fp32 this value would first
    # round to the midpoint and then (half-even) down: a double rounding.
    above = 1.0 + 2.0 ** -11 + 2.0 ** -40
    assert np.float32(above) == np.float32(1.0 + 2.0 ** -11)
    assert fp.fp16_rne(above) == 1.0 + 2.0 ** -10
    # 3 * 2^-11 (midpoint above an odd mantissa) rounds up to even
    assert fp.fp16_rne(1.0 + 3 * 2.0 ** -11) == 1.0 + 2 * 2.0 ** -10
    # overflow threshold
    assert fp.fp16_rne(65504.0) == 65504.0
    assert fp.fp16_rne(65519.999) == 65504.0
    assert math.isinf(fp.fp16_rne(65520.0))
    # subnormals: quantum 2^-24, midpoint 1.5 * 2^-24 goes to even (2 * 2^-24)
    assert fp.fp16_rne(1.5 * 2.0 ** -24) == 2 * 2.0 ** -24
    assert fp.fp16_rne(0.5 * 2.0 ** -24) == 0.0
    assert fp.fp16_bits(1.0) == 0x3C00


def test_bf16_rne_matches_torch_on_fp32_inputs():
    rng = np.random.default_rng(5)
    v32 = (rng.standard_normal(20000) * 2.0).astype(np.float32)
    lib = torch.from_numpy(v32).to(torch.bfloat16).to(torch.float64).numpy()
    mine = np.array([fp.bf16_rne(float(v)) for v in v32])
    assert np.array_equal(lib, mine)
    assert fp.bf16_rne(1.0 + 2.0 ** -8) == 1.0            # midpoint -> even
    assert fp.bf16_rne(1.0 + 2.0 ** -8 + 2.0 ** -30) == 1.0 + 2.0 ** -7
