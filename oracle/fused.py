"""What the fused forms of the product compute, for the "Module ops" entries
w4a16_gemv_silu_input (the activation is silu(gate) * up, per element, inside
the kernel) and w4a16_gemv_qg / w4a16_gemv_qkvz (rows that interleave parts
per head or group, stored de-interleaved).

TEST INFRASTRUCTURE ONLY (see the oracle package docstring).

Reading of the pages: the kernel's activation is a bf16 vector (it feeds a
bf16 matrix product), so silu(gate) * up is rounded once to bf16, to nearest,
ties to even; here silu(g) = g / (1 + exp(-g)) and the product with u are
evaluated in float64 before that one rounding.  The de-interleaved output
puts, for parts p = 0, 1, ..., every group's rows of part p together, groups
in order: [part 0 of all groups | part 1 of all groups | ...].
"""
from __future__ import annotations

import numpy as np

from .expand import round_to_bf16
from .linear import bf16_bits_to_f64


def silu(g: np.ndarray) -> np.ndarray:
    """g / (1 + exp(-g)) in float64 (exp overflowing to inf gives -0 or 0)."""
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def silu_mul_bf16(gate_bits: np.ndarray, up_bits: np.ndarray) -> np.ndarray:
    """bf16 bits of silu(gate) * up, rounded once from float64."""
    return round_to_bf16(silu(bf16_bits_to_f64(gate_bits)) * bf16_bits_to_f64(up_bits))


def deinterleave_columns(n: int, widths) -> np.ndarray:
    """Output column of each weight row: row r of part p of group g goes to
    groups * (widths[0] + .. + widths[p-1]) + g * widths[p] + r."""
    widths = [int(w) for w in widths]
    gw = sum(widths)
    if n % gw:
        raise ValueError("N must be a whole number of groups")
    groups = n // gw
    out = np.empty(n, dtype=np.int64)
    for g in range(groups):
        before = 0
        for p, w in enumerate(widths):
            for r in range(w):
                out[g * gw + before + r] = groups * before + g * w + r
            before += w
    return out


def deinterleave(y_rows_by_weight_row: np.ndarray, widths) -> np.ndarray:
    """y[M, N] indexed by weight row -> the de-interleaved y[M, N]."""
    y = np.asarray(y_rows_by_weight_row)
    cols = deinterleave_columns(y.shape[1], widths)
    out = np.empty_like(y)
    out[:, cols] = y
    return out
