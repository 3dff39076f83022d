"""Per-token symmetric int8 activations after the group FWHT (oracle).

Test infrastructure only.  Needle .cact/W4A8 article, section 1: the
configuration is W4A8, 8-bit activations; section 4 quantizes queries per
head with symmetric A8.  The CQ reconstruction (section 1) multiplies the
codebook vector by the orthogonal H, so dot(w_g, x_g) can be taken in the
rotated domain: dot(w_g, x_g) = norm_g/G * dot(cb[idx_g], H_u x_g).  The
activation is therefore rotated, not the weights.

Readings taken: one scale per token (row), range +-127, round half to even
(as the Minueza page's Q4_0 code uses np.rint), quantizing the rotated
values x_u = H_u x_g (unnormalized), s = max|x_u| / 127 over the whole row
(s = 1 for an all-zero row), q = clip(rint(x_u / s), -127, 127).

Two modes: ``fp32`` performs every step in fp32 with the same butterfly
network and a correctly rounded fp32 division, so its q is the one and only
right answer for a device that does the same; ``fp64`` is the exact math.

``act_quant_a8_unrotated`` is the same per-token quantizer without the
rotation, for the Q4_0 format, which carries no Hadamard rotation (the
Minueza-32M -> KMCU v1 page, sections 2-3): its group is 1, and the
transform of length 1 is the identity.
"""
from __future__ import annotations

import numpy as np

from .hadamard import fwht_u

QMAX = 127


def act_quant_a8(x: np.ndarray, group: int, mode: str = "fp32"):
    """x fp32 [m, k] -> (q int8 [m, k], scale fp32 [m] or fp64 in fp64 mode)."""
    x = np.asarray(x, dtype=np.float32)
    m, k = x.shape
    if k % group:
        raise ValueError("k must be a multiple of group")
    if mode == "fp32":
        dt = np.float32
    elif mode == "fp64":
        dt = np.float64
    else:
        raise ValueError("mode is fp32 or fp64")
    u = fwht_u(x.astype(dt).reshape(m, k // group, group), dtype=dt).reshape(m, k)
    amax = np.max(np.abs(u), axis=1)
    s = np.where(amax > 0, amax / dt(QMAX), dt(1.0)).astype(dt)
    r = np.rint(u / s[:, None])          # division in dt, correctly rounded
    q = np.clip(r, -QMAX, QMAX).astype(np.int8)
    return q, s


def act_quant_a8_unrotated(x: np.ndarray, mode: str = "fp32"):
    """Per-token symmetric int8 of x itself: s = max|x| / 127 over the row
    (1 for an all-zero row), q = clip(rint(x / s), -127, 127)."""
    return act_quant_a8(x, 1, mode)


def dequant_a8(q: np.ndarray, s: np.ndarray, group: int) -> np.ndarray:
    """Activation the int8 codes stand for, fp64: x_hat_g = s * H_u q_g / G."""
    q = np.asarray(q, dtype=np.float64)
    m, k = q.shape
    u = fwht_u(q.reshape(m, k // group, group)).reshape(m, k)
    return u * (np.asarray(s, dtype=np.float64)[:, None] / group)
