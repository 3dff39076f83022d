"""Walsh-Hadamard transform (oracle; test infrastructure only).

Needle .cact/W4A8 article, section 1: each 128-wide group of a weight row is
rotated by a *normalized* Walsh-Hadamard transform before quantization, and
the reconstruction multiplies by that same normalized matrix H.

Reading taken here (the page does not name an ordering): Sylvester natural
order, ``H_1 = [1]``, ``H_2n = [[H_n, H_n], [H_n, -H_n]]``.  ``H_u`` is the
unnormalized +-1 matrix and ``H = H_u / sqrt(G)``, which is symmetric and its
own inverse.
"""
from __future__ import annotations

import numpy as np


def sylvester(g: int) -> np.ndarray:
    """Unnormalized Sylvester Hadamard matrix H_u of order g (int64 +-1)."""
    if g < 1 or (g & (g - 1)) != 0:
        raise ValueError("Hadamard order must be a power of two")
    h = np.ones((1, 1), dtype=np.int64)
    while h.shape[0] < g:
        h = np.block([[h, h], [h, -h]])
    return h


def fwht_u(x: np.ndarray, dtype=np.float64) -> np.ndarray:
    """Unnormalized fast Walsh-Hadamard transform along the last axis.

    Butterfly stages run with half-width h = 1, 2, 4, ..., G/2.  At each
    stage every pair (j, j+h) with ``j mod 2h < h`` becomes (a+b, a-b),
    where a is the value at j and b the value at j+h.  The arithmetic is done
    in ``dtype`` (fp64 by default; fp32 reproduces an fp32 butterfly of the
    same network exactly).  Equals ``x @ sylvester(G)`` up to rounding.
    """
    v = np.array(x, dtype=dtype, copy=True)
    g = v.shape[-1]
    if g < 1 or (g & (g - 1)) != 0:
        raise ValueError("FWHT length must be a power of two")
    lead = v.shape[:-1]
    h = 1
    while h < g:
        blk = v.reshape(lead + (g // (2 * h), 2, h))
        a = blk[..., 0, :].copy()
        b = blk[..., 1, :].copy()
        blk[..., 0, :] = a + b
        blk[..., 1, :] = a - b
        v = blk.reshape(lead + (g,))
        h *= 2
    return v


def fwht(x: np.ndarray) -> np.ndarray:
    """Normalized transform H x = H_u x / sqrt(G), in fp64."""
    g = np.shape(x)[-1]
    return fwht_u(x) / np.sqrt(np.float64(g))
