"""Seeded synthetic inputs for the quantized-matmul workloads.

This module only draws random numbers and arranges them into the shapes the
workloads use.  It holds none of the quantization arithmetic, so both the
HIP path and the CPU oracle can be fed from it without sharing any of the
method's code.  Everything is drawn with ``numpy.random.default_rng(seed)``
(PCG64) in fp64 and cast to fp32 where the workload is fp32.

Workload recipes (weights are 0.02*N(0,1), activations N(0,1)):

* ``cq_single``: one 512x512 matrix, batch-1 activation (the Needle CQ
  W4A8 article, section 1: 4-bit weights, 8-bit activations, group 128).
* ``minueza_q4_0_pass``: the ten-layer Minueza-32M projection shapes plus the
  tied 32002x312 head (the Minueza/KMCU page, section 1: dim 312, 4 kv heads
  of 26, ffn 1092, vocab 32002; --force-tie).  One activation per matrix,
  drawn after all weights.
* ``cq_decode_8b``: 8B-class layer shapes 4096x4096, 1024x4096, 14336x4096,
  4096x14336 with 1% outlier rows scaled by 8, batch-1 activations.
* ``cq_prefill``: 512 tokens x 4096 activations, weights 14336x4096 and
  4096x4096 without outliers.
* ``cq_bit_sweep``: one 14336x4096 matrix with 1% outlier rows, activations
  for batch 1, 4 and 16.
* ``weight_matrix_mixed`` (parity tests): 0.02*N(0,1) rows among which every
  7th row is scaled by 1e-3, every 11th by 1e-4, every 13th by 1e-6, one row
  has its groups alternately scaled by 1 and 1e-4, and one row is all zero,
  so that group norms span fp16 from its normal range deep into its
  subnormals within one matrix.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

WEIGHT_STD = 0.02
OUTLIER_FRACTION = 0.01
OUTLIER_SCALE = 8.0

# Minueza-32M projection shapes, [out, in], in the order they are drawn.
MINUEZA_LAYER_SHAPES = (
    ("q", 312, 312),
    ("k", 104, 312),
    ("v", 104, 312),
    ("o", 312, 312),
    ("gate", 1092, 312),
    ("up", 1092, 312),
    ("down", 312, 1092),
)
MINUEZA_LAYERS = 10
MINUEZA_HEAD = ("head", 32002, 312)

DECODE_8B_SHAPES = ((4096, 4096), (1024, 4096), (14336, 4096), (4096, 14336))
PREFILL_TOKENS = 512
PREFILL_SHAPES = ((14336, 4096), (4096, 4096))
SWEEP_SHAPE = (14336, 4096)
SWEEP_BATCHES = (1, 4, 16)


def rng_for(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def gaussian_samples(n: int = 400_000, seed: int = 0) -> np.ndarray:
    """fp64 N(0,1) draws for the codebook fit (400k samples on the pages)."""
    return rng_for(seed).standard_normal(n)


def weight_matrix(rng: np.random.Generator, rows: int, cols: int,
                  outliers: bool = False, std: float = WEIGHT_STD) -> np.ndarray:
    """fp32 ``std*N(0,1)`` matrix; with ``outliers`` ceil(1%) rows are x8."""
    w = (std * rng.standard_normal((rows, cols))).astype(np.float32)
    if outliers:
        n_out = int(math.ceil(OUTLIER_FRACTION * rows))
        sel = rng.choice(rows, n_out, replace=False)
        w[sel] *= np.float32(OUTLIER_SCALE)
    return w


MIXED_ROW_SCALES = ((7, 1e-3), (11, 1e-4), (13, 1e-6))


def weight_matrix_mixed(rng: np.random.Generator, rows: int, cols: int, group: int = 128,
                        outliers: bool = False) -> np.ndarray:
    """``weight_matrix`` with rows at very different scales (see the module notes):
    rows r with r % p == p - 1 scaled by f for each (p, f) of MIXED_ROW_SCALES
    (later entries win), row 1 with its odd groups scaled by 1e-4 (when there is
    more than one group) and row rows // 2 set to zero."""
    w = weight_matrix(rng, rows, cols, outliers=outliers)
    r = np.arange(rows)
    for period, f in MIXED_ROW_SCALES:
        w[r % period == period - 1] *= np.float32(f)
    if rows > 1 and cols > group:
        g = w[1, :cols // group * group].reshape(-1, group)       # whole groups (a view of row 1)
        g[1::2] *= np.float32(1e-4)
    w[rows // 2] = 0.0
    return w


def activations(rng: np.random.Generator, batch: int, cols: int) -> np.ndarray:
    return rng.standard_normal((batch, cols)).astype(np.float32)


@dataclass
class Workload:
    name: str
    weights: list = field(default_factory=list)      # list of (label, fp32 [out,in])
    acts: list = field(default_factory=list)         # list of fp32 [batch, in]


def cq_single(seed: int = 0) -> Workload:
    rng = rng_for(seed)
    w = weight_matrix(rng, 512, 512)
    x = activations(rng, 1, 512)
    return Workload("cq_single_512x512_b1", [("w", w)], [x])


def minueza_q4_0_pass(seed: int = 0, layers: int = MINUEZA_LAYERS) -> Workload:
    rng = rng_for(seed)
    wl = Workload(f"minueza_q4_0_pass_{layers}L_tied_head")
    for layer in range(layers):
        for lab, r, c in MINUEZA_LAYER_SHAPES:
            wl.weights.append((f"L{layer}.{lab}", weight_matrix(rng, r, c)))
    lab, r, c = MINUEZA_HEAD
    wl.weights.append((lab, weight_matrix(rng, r, c)))
    for _, w in wl.weights:
        wl.acts.append(activations(rng, 1, w.shape[1]))
    return wl


def cq_decode_8b(seed: int = 0, shapes=DECODE_8B_SHAPES) -> Workload:
    rng = rng_for(seed)
    wl = Workload("cq_w4a8_decode_8b_layers_b1")
    for (n, k) in shapes:
        wl.weights.append((f"{n}x{k}", weight_matrix(rng, n, k, outliers=True)))
    for _, w in wl.weights:
        wl.acts.append(activations(rng, 1, w.shape[1]))
    return wl


def cq_prefill(seed: int = 0, tokens: int = PREFILL_TOKENS, shapes=PREFILL_SHAPES) -> Workload:
    rng = rng_for(seed)
    wl = Workload(f"cq_w4a8_prefill_m{tokens}")
    x = activations(rng, tokens, shapes[0][1])
    for (n, k) in shapes:
        wl.weights.append((f"{n}x{k}", weight_matrix(rng, n, k)))
    wl.acts.append(x)
    return wl


def cq_bit_sweep(seed: int = 0, shape=SWEEP_SHAPE, batches=SWEEP_BATCHES) -> Workload:
    rng = rng_for(seed)
    n, k = shape
    wl = Workload(f"cq_bit_sweep_{n}x{k}")
    wl.weights.append((f"{n}x{k}", weight_matrix(rng, n, k, outliers=True)))
    for b in batches:
        wl.acts.append(activations(rng, b, k))
    return wl
