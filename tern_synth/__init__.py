"""Seeded synthetic inputs for the ternary-weight linear layer.

This module only draws random inputs; it holds none of the layer's
arithmetic (no quantisation, no packing, no contraction). Both sides use it:
the tests feed the same arrays to the CPU oracle and to the HIP library, and
``bench.py`` draws its device inputs from it.

Recipe (numpy ``default_rng``, PCG64), one weight stream per matrix and one
activation stream per (matrix, T):

* weights ``w`` int8 ``[N, K]``, iid: P(-1) = P(0) = P(+1) = 1/3 for the
  small 256 -> 128 case, P(0) = 0.4 and P(+1) = P(-1) = 0.3 otherwise;
* scales: one per group of ``G`` consecutive weights along K, drawn
  U(0.01, 0.05) in fp64 and rounded to fp16 (nearest even);
* outlier channels: ``round(0.01 * K)`` distinct input channels per matrix
  (none in the small case), the same for every token;
* activations ``x``: N(0, 1) in fp32, outlier channels multiplied by 20,
  rounded to bf16 (nearest even).

Draw order on the weight stream: w, scales, outlier channels. The activation
stream draws x only.
"""
from __future__ import annotations

import dataclasses

import numpy as np


@dataclasses.dataclass(frozen=True)
class Shape:
    name: str
    k: int  # input features (K)
    n: int  # output features (N)
    group: int  # scale group size along K (G)
    p_zero: float  # P(w == 0); P(+1) = P(-1) = (1 - p_zero) / 2
    outliers: bool  # 1 % of input channels scaled x20
    seed: int  # weight-stream seed


# The layer shapes of the workloads (27B-class decoder, K in -> N out).
SMALL = Shape("small_256x128", 256, 128, 64, 1.0 / 3.0, False, 101)
GATE_UP = Shape("gate_up_5120x34816", 5120, 34816, 128, 0.4, True, 201)
DOWN = Shape("down_17408x5120", 17408, 5120, 128, 0.4, True, 202)
OUT_PROJ = Shape("o_proj_5120x5120", 5120, 5120, 128, 0.4, True, 203)

SHAPES = {s.name: s for s in (SMALL, GATE_UP, DOWN, OUT_PROJ)}

# One decoder layer of the 64-layer stack: q, k, v, o (5120x5120), gate and up
# (5120 -> 17408 each), down (17408 -> 5120).
STACK_LAYERS = 64
STACK_PROJ = (("q", 5120, 5120), ("k", 5120, 5120), ("v", 5120, 5120), ("o", 5120, 5120),
              ("gate", 5120, 17408), ("up", 5120, 17408), ("down", 17408, 5120))


def stack_shape(layer: int, proj: int) -> Shape:
    name, k, n = STACK_PROJ[proj]
    return Shape(f"L{layer}.{name}", k, n, 128, 0.4, True, 5000 + 10 * layer + proj)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest even), returned as uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + r) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return np.asarray(b, dtype=np.uint16).view(np.float16).astype(np.float32)


def draw_weights(rng: np.random.Generator, n: int, k: int, p_zero: float,
                 chunk_rows: int = 2048) -> np.ndarray:
    """iid ternary weights, int8 [n, k]."""
    w = np.empty((n, k), np.int8)
    p_neg = np.float32((1.0 - p_zero) / 2.0)
    p_pos_lo = np.float32(1.0 - (1.0 - p_zero) / 2.0)
    for r0 in range(0, n, chunk_rows):
        r1 = min(n, r0 + chunk_rows)
        u = rng.random((r1 - r0, k), dtype=np.float32)
        blk = (u >= p_pos_lo).astype(np.int8)
        blk -= (u < p_neg).astype(np.int8)
        w[r0:r1] = blk
    return w


def draw_scales(rng: np.random.Generator, n: int, k: int, group: int) -> np.ndarray:
    """U(0.01, 0.05) per (row, group), as fp16 bits uint16 [n, k // group]."""
    s = rng.uniform(0.01, 0.05, size=(n, k // group))
    return s.astype(np.float16).view(np.uint16)


@dataclasses.dataclass
class Weights:
    shape: Shape
    w: np.ndarray  # int8 [N, K]
    s: np.ndarray  # fp16 bits [N, K // G]
    outlier_channels: np.ndarray  # int64 [round(0.01 K)] (empty when none)


def weights(shape: Shape) -> Weights:
    rng = np.random.default_rng(shape.seed)
    w = draw_weights(rng, shape.n, shape.k, shape.p_zero)
    s = draw_scales(rng, shape.n, shape.k, shape.group)
    n_out = int(round(0.01 * shape.k)) if shape.outliers else 0
    ch = np.sort(rng.choice(shape.k, size=n_out, replace=False)) if n_out else np.zeros(0, np.int64)
    return Weights(shape, w, s, ch.astype(np.int64))


def activations(wts: Weights, T: int, salt: int = 0) -> np.ndarray:
    """bf16 bits uint16 [T, K] for this matrix and token count."""
    rng = np.random.default_rng([wts.shape.seed, 1, T, salt])
    x = rng.standard_normal((T, wts.shape.k), dtype=np.float32)
    if wts.outlier_channels.size:
        x[:, wts.outlier_channels] *= np.float32(20.0)
    return f32_to_bf16_bits(x)


def integer_activations(K: int, T: int, seed: int, lo: int = -8, hi: int = 8) -> np.ndarray:
    """bf16 bits of small integers: every product and sum in fp32 is exact."""
    rng = np.random.default_rng([seed, 2, T])
    return f32_to_bf16_bits(rng.integers(lo, hi + 1, size=(T, K)).astype(np.float32))


def pow2_scales(n: int, k: int, group: int, seed: int, lo: int = -6, hi: int = -2) -> np.ndarray:
    """fp16 bits of powers of two 2^e, e in [lo, hi]."""
    rng = np.random.default_rng([seed, 3])
    e = rng.integers(lo, hi + 1, size=(n, k // group))
    return np.ldexp(np.ones_like(e, dtype=np.float64), e).astype(np.float16).view(np.uint16)
