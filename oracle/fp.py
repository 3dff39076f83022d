"""Exact rounding helpers for the oracle (test infrastructure only).

The CQ format stores each group's L2 norm as FP16 (Needle .cact/W4A8 article,
section 1; the mmap article restates it).  The oracle rounds the fp64 norm to
fp16 directly, round-half-to-even, without passing through fp32 (one
rounding, not two).  The shipped codebook is rounded to bfloat16-representable
values the same way (a reading: the pages do not state the codebook's
precision).
"""
from __future__ import annotations

import math

import numpy as np

FP16_MAX = 65504.0


def _round_sig_rne(x: float, sig_bits: int, min_exp: int) -> float:
    """Round a finite fp64 ``x`` to ``sig_bits`` significant bits, half-even.

    ``min_exp`` is the exponent (as from ``math.frexp``) below which the
    format becomes subnormal; there the quantum stays fixed at
    2**(min_exp - sig_bits).  Exact: frexp/ldexp scale by powers of two and
    Python's round() on a float rounds the exact binary value half-to-even.
    """
    if x == 0.0 or not math.isfinite(x):
        return x
    m, e = math.frexp(x)            # x = m * 2**e, 0.5 <= |m| < 1
    e_eff = max(e, min_exp)
    scaled = math.ldexp(x, sig_bits - e_eff)   # exact (power-of-two scaling)
    r = round(scaled)                          # half-to-even on exact value
    return math.ldexp(float(r), e_eff - sig_bits)


def fp16_rne(x: float) -> float:
    """fp64 -> nearest fp16 value (as a Python float); inf on overflow."""
    # fp16: 11 significant bits; smallest normal 2**-14 = 0.5 * 2**-13.
    r = _round_sig_rne(float(x), 11, -13)
    if abs(r) > FP16_MAX:
        return math.copysign(math.inf, r)
    return r


def fp16_bits(x: float) -> int:
    """Bit pattern (uint16) of ``fp16_rne(x)``."""
    return int(np.array(fp16_rne(x), dtype=np.float16).view(np.uint16))


def bf16_rne(x: float) -> float:
    """fp64 -> nearest bfloat16 value (8 significant bits), half-even."""
    # bf16 shares fp32's exponent range; the codebook never goes near it.
    return _round_sig_rne(float(x), 8, -125)
