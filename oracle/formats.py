"""Decode tables of the two NVFP4 element formats, built from their bit fields.

e2m1 (4 bits: sign, 2 exponent bits with bias 1, 1 mantissa bit) is the weight
element named in "10 Kernels" section 10.2 and in the "Module ops" entries
``w4a16_gemm`` and ``w4a16_tc_rows``.  The pages name the format but print no
values; its bit layout is the OCP Microscaling Formats v1.0 FP4 (E2M1) one.

e4m3 (8 bits: sign, 4 exponent bits with bias 7, 3 mantissa bits, no
infinities, NaN when all exponent and mantissa bits are set) is the group-scale
format of the same entries; "Module ops" constant ``E4M3_MAX`` is its largest
finite magnitude.  This is the OCP 8-bit floating point "E4M3" variant.
"""
from __future__ import annotations

import math

import numpy as np


def e2m1_value(code: int) -> float:
    """Value of one 4-bit e2m1 code."""
    sign = -1.0 if (code >> 3) & 1 else 1.0
    exponent = (code >> 1) & 3
    mantissa = code & 1
    if exponent == 0:                       # subnormal: 0 or 0.5
        magnitude = mantissa * 0.5
    else:
        magnitude = (1.0 + mantissa / 2.0) * 2.0 ** (exponent - 1)
    return sign * magnitude


def e4m3_value(byte: int) -> float:
    """Value of one e4m3 byte (NaN for the two NaN encodings)."""
    sign = -1.0 if (byte >> 7) & 1 else 1.0
    exponent = (byte >> 3) & 15
    mantissa = byte & 7
    if exponent == 15 and mantissa == 7:
        return math.nan
    if exponent == 0:                       # subnormal
        magnitude = (mantissa / 8.0) * 2.0 ** -6
    else:
        magnitude = (1.0 + mantissa / 8.0) * 2.0 ** (exponent - 7)
    return sign * magnitude


E2M1 = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
E4M3 = np.array([e4m3_value(b) for b in range(256)], dtype=np.float64)
E2M1.setflags(write=False)
E4M3.setflags(write=False)
