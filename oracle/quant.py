"""Reference quantiser fp32 W[N, K] -> NVFP4 (packed e2m1, e4m3 group scales, t).

The pages fix the stored format (see ``oracle.linear``) but not how a packer
chooses the scales; "Module ops" ``quantize_bf16_to_nvfp4`` only shows a packer
that writes packed e2m1 [M, K/2] plus one e4m3 scale per 16 elements.  The
reading used here, every step in IEEE float64 in this order:

Q1  amax_T = max |W| (non-finite W is an error);
    t = fp32(amax_T / (6 * 448)), and t = 1 when amax_T or t is 0, so that the
    largest group scale lands on E4M3_MAX = 448 ("Module ops" constant);
Q2  per row n and group g of 16 consecutive k: a = max |W[n, 16g:16g+16]|,
    u = (a / 6) / t, i.e. the group's absmax over the largest e2m1 magnitude;
Q3  s = e4m3 code nearest to u, ties to the even code, u >= 448 -> 0x7E;
Q4  S = E4M3[s] * t (exact); a group with S == 0 gets all-zero codes;
Q5  v = W / S; c = e2m1 code nearest to |v|, ties to the even code, |v| > 6
    saturates to 6; the sign bit is set when v < 0 and the magnitude code is
    not 0;
Q6  byte j of a row = c[2j] | c[2j+1] << 4 (low nibble = even k).

Round-to-nearest with saturation to the largest finite value is what the
conversion named on "CUDA Kernel Engineering" (SM121 hardware budget, the
native FP4 caveat) does for e2m1; the same rule is used for e4m3.
"""
from __future__ import annotations

import numpy as np

from .formats import E2M1, E4M3

GROUP = 16
E4M3_MAX = 448.0
E2M1_MAX = 6.0
E4M3_POSITIVE = E4M3[:0x7F]          # codes 0x00..0x7E, increasing
E2M1_POSITIVE = E2M1[:8]             # codes 0..7, increasing


def _nearest_code(values: np.ndarray, grid: np.ndarray) -> np.ndarray:
    """Index of the nearest grid point to each value (all >= 0, grid increasing).

    Ties go to the even index; values above the last point take the last index."""
    values = np.asarray(values, dtype=np.float64)
    hi = np.searchsorted(grid, values, side="left")      # grid[hi-1] < v <= grid[hi]
    hi = np.clip(hi, 0, len(grid) - 1)
    lo = np.clip(hi - 1, 0, len(grid) - 1)
    d_lo = np.abs(values - grid[lo])
    d_hi = np.abs(grid[hi] - values)
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    return np.where(values >= grid[-1], len(grid) - 1, code)


def e4m3_round(u: np.ndarray) -> np.ndarray:
    """Q3: non-negative finite u -> e4m3 code (uint8), RNE, saturating at 0x7E."""
    return _nearest_code(u, E4M3_POSITIVE).astype(np.uint8)


def e2m1_round(v: np.ndarray) -> np.ndarray:
    """Q5: finite v -> e2m1 code (uint8), RNE on |v|, saturating at 6, signed."""
    v = np.asarray(v, dtype=np.float64)
    mag = _nearest_code(np.abs(v), E2M1_POSITIVE).astype(np.uint8)
    sign = ((v < 0) & (mag != 0)).astype(np.uint8) << 3
    return mag | sign


def tensor_scale(w: np.ndarray) -> float:
    """Q1."""
    w64 = np.asarray(w, dtype=np.float32).astype(np.float64)
    if not np.all(np.isfinite(w64)):
        raise ValueError("non-finite weight")
    amax = float(np.max(np.abs(w64))) if w64.size else 0.0
    t = float(np.float32(amax / (E2M1_MAX * E4M3_MAX)))
    if amax == 0.0 or t == 0.0:
        t = 1.0
    return t


def quantize_ref(w: np.ndarray) -> tuple[np.ndarray, np.ndarray, float]:
    """fp32 W[N, K] (K % 16 == 0) -> (packed [N, K/2] u8, scales [N, K/16] u8, t)."""
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    if k % GROUP:
        raise ValueError("K must be a multiple of 16")
    t = tensor_scale(w)
    groups = w.astype(np.float64).reshape(n, k // GROUP, GROUP)
    a = np.max(np.abs(groups), axis=2)                       # Q2
    u = (a / E2M1_MAX) / t
    s = e4m3_round(u)                                        # Q3
    big_s = E4M3[s] * t                                      # Q4
    safe = np.where(big_s == 0.0, 1.0, big_s)
    v = groups / safe[:, :, None]                            # Q5
    codes = e2m1_round(v)
    codes[big_s == 0.0] = 0
    codes = codes.reshape(n, k)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)   # Q6
    return packed, s.astype(np.uint8), t
