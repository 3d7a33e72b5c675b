"""The NVFP4 weight expanded to bf16, for the expand-then-multiply regime of
"10 Kernels" 10.2 and the "Module ops" entry dequant_nvfp4_to_bf16 (an NVFP4
weight [n, k] dequantised to BF16 [n, k], with the per-tensor scale).

TEST INFRASTRUCTURE ONLY (see the oracle package docstring).

bf16 has 8 significant bits, an 8-bit exponent (bias 127) and subnormals
below 2^-126 with quantum 2^-133.  Rounding is to the nearest value, ties to
the even significand, written out here from that definition on exact float64
inputs.
"""
from __future__ import annotations

import numpy as np

from .linear import dequant

BF16_MIN_NORMAL_EXP = -126
BF16_MANT_BITS = 7


def round_to_bf16(v: np.ndarray) -> np.ndarray:
    """float64 -> nearest bf16 (ties to even), as uint16 bit patterns.

    The value is split as an integer multiple of the bf16 quantum of its
    binade (2^(e - 7) for |v| in [2^e, 2^(e+1)), 2^-133 below 2^-126); the
    multiple is rounded to the nearest integer, ties to even (numpy.rint), and
    the result re-encoded.  Exact for every finite float64 input whose rounded
    magnitude stays below 2^128; NaN maps to the quiet NaN 0x7FC0."""
    v = np.asarray(v, dtype=np.float64)
    out = np.zeros(v.shape, dtype=np.uint16)
    nan = np.isnan(v)
    a = np.abs(np.where(nan, 0.0, v))
    sign = (np.signbit(v) & ~nan).astype(np.uint16) << 15
    nz = a > 0
    e = np.zeros(v.shape, dtype=np.int64)
    e[nz] = np.floor(np.log2(a[nz])).astype(np.int64)
    # np.log2 may land one off at exact powers of two: fix the binade exactly
    e = np.where(nz & (np.ldexp(1.0, e) > a), e - 1, e)
    e = np.where(nz & (np.ldexp(1.0, e + 1) <= a), e + 1, e)
    q_exp = np.maximum(e, BF16_MIN_NORMAL_EXP) - BF16_MANT_BITS
    mult = np.rint(np.ldexp(a, -q_exp))                      # exact scaling, then ties-to-even
    r = np.ldexp(mult, q_exp)                                 # the rounded magnitude (exact)
    # encode r: normal if r >= 2^-126 (rounding may carry into the next binade)
    normal = r >= np.ldexp(1.0, BF16_MIN_NORMAL_EXP)
    re = np.zeros(v.shape, dtype=np.int64)
    re[normal] = np.floor(np.log2(r[normal])).astype(np.int64)
    re = np.where(normal & (np.ldexp(1.0, re) > r), re - 1, re)
    re = np.where(normal & (np.ldexp(1.0, re + 1) <= r), re + 1, re)
    bits = np.zeros(v.shape, dtype=np.int64)
    sub = ~normal
    bits[sub] = np.ldexp(r[sub], -(BF16_MIN_NORMAL_EXP - BF16_MANT_BITS)).astype(np.int64)
    mant_n = (np.ldexp(r[normal], -re[normal]) * 2 ** BF16_MANT_BITS).astype(np.int64) - 2 ** BF16_MANT_BITS
    bits[normal] = ((re[normal] + 127) << BF16_MANT_BITS) | mant_n
    bits = np.where(normal & (re > 127), 0x7F80, bits)        # overflow to infinity
    out[:] = (bits.astype(np.uint16) | sign)
    out[nan] = 0x7FC0
    return out


def dequant_bf16(w_packed: np.ndarray, scales: np.ndarray, t: float, apply_tensor_scale: bool) -> np.ndarray:
    """[n, k/2] packed e2m1 and [n, k/16] e4m3 -> bf16 bits [n, k]: the exact
    t * e4m3 * e2m1 (or e4m3 * e2m1 without t), rounded once to bf16."""
    wd = dequant(w_packed, scales, float(t) if apply_tensor_scale else 1.0)
    return round_to_bf16(wd)
