"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle.

This module draws random numbers and casts them to the storage types the
product takes (fp32 weights before packing, bf16 activations).  It holds none
of the NVFP4 arithmetic: no decoding, no quantisation, no products.  Both the
oracle and the HIP path receive the bytes made here, so the two sides never
generate their own inputs.

Every generator is ``numpy.random.Generator(PCG64(seed))``.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

WEIGHT_STD = 0.02          # weights are N(0, 0.02) in fp32 before packing
OUTLIER_FRACTION = 0.01    # the QKV-style workload scales 1 % of x by 50
OUTLIER_SCALE = 50.0


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest, ties to even); return the uint16 bits.

    Non-finite inputs keep their class (NaN stays NaN, inf stays inf)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    nan = np.isnan(a)
    out = rounded.astype(np.uint16)
    out[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)   # keep a quiet NaN
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bits to fp32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def weights_f32(n: int, k: int, seed: int, std: float = WEIGHT_STD) -> np.ndarray:
    """W[n, k] = std * N(0, 1), drawn in fp32."""
    w = rng(seed).standard_normal((n, k), dtype=np.float32)
    w *= np.float32(std)
    return w


def activations_bf16(m: int, k: int, seed: int, outliers: bool = False) -> np.ndarray:
    """x[m, k] as bf16 bits: N(0, 1) drawn in fp32, optionally with 1 % of the
    entries (chosen by U[0,1) < 0.01 from the same generator) multiplied by 50 in
    fp32, then one round-to-nearest-even cast to bf16."""
    g = rng(seed)
    x = g.standard_normal((m, k), dtype=np.float32)
    if outliers:
        mask = g.random((m, k), dtype=np.float32) < OUTLIER_FRACTION
        x[mask] *= np.float32(OUTLIER_SCALE)
    return f32_to_bf16_bits(x)


def random_codes(n: int, k: int, seed: int) -> tuple[np.ndarray, np.ndarray]:
    """Uniform random packed nibbles [n, k/2] and valid scale bytes [n, k/16].

    Scale bytes are drawn from 0x00..0x7E: non-negative, never NaN."""
    g = rng(seed)
    packed = g.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    scales = g.integers(0, 0x7F, size=(n, k // 16), dtype=np.uint8)
    return packed, scales


@dataclass(frozen=True)
class Shape:
    n: int
    k: int


# Workloads shaped like the pages' decode and verify products.
SINGLE = Shape(1024, 1024)                     # one small linear, M = 1
INVARIANCE = Shape(4096, 4096)                 # row-invariance sweep, M = 1..32
QKV = Shape(12288, 4096)                       # fused QKV-style, M = 16 and 17..32
HEAD = Shape(151552, 4096)                     # output head, fp32 logits
ROUND_LAYERS = 48
ROUND_SHAPES = (Shape(8192, 4096), Shape(4096, 8192),
                Shape(24576, 4096), Shape(4096, 12288))
ROUND_M = (1, 8, 16, 32)

SEEDS = {
    "single": (11, 12),
    "invariance": (21, 22),
    "qkv": (31, 32),
    "head": (51, 52),
}


def round_weight_seed(layer: int, proj: int) -> int:
    return 4000 + 4 * layer + proj


def round_act_seed(layer: int, proj: int, m: int) -> int:
    return 5000 + 4 * layer + proj + 1000 * m


def round_weight_bytes() -> int:
    """Packed nibbles plus scale bytes of one decode round (48 layers)."""
    per_layer = sum(s.n * s.k // 2 + s.n * s.k // 16 for s in ROUND_SHAPES)
    return ROUND_LAYERS * per_layer
