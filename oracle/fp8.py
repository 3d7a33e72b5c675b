"""FP8 block-scaled weight-only product (W8A16), the pages' second weight
format: "10 Kernels" 10.3 (block-scaled FP8 read as stored; the tile is 128
wide along K, so each step covers one scale block and the scale is one number
applied to the fp32 sum) and "Module ops" w8a16_gemm (C[M,N] = A[M,K] @
dequant(B[N,K])^T with the FP32 block scale [ceil(N/128), ceil(K/128)]).

TEST INFRASTRUCTURE ONLY (see the oracle package docstring).

    y[m, n] = sum_k x[m, k] * E4M3(B[n, k]) * S[n // 128, k // 128]

Every weight E4M3(B) * S has at most 4 + 24 significant bits, so the
dequantised matrix is exact in float64 and y_ref adds K exact products with a
BLAS dgemm, as oracle.linear does for NVFP4.

The pages store checkpoints already quantised; the synthetic weights here need
a quantiser, and its rule is this reading: per 128 x 128 block,
S = fp32(max|W| / 448) (1 when that is 0), codes = E4M3 of W / S rounded to
nearest, ties to even, saturating at 448, in IEEE float64 in that order.
"""
from __future__ import annotations

import numpy as np

from .formats import E4M3
from .linear import bf16_bits_to_f64
from .quant import e4m3_round

BLOCK = 128
E4M3_MAX = 448.0


def dequant_fp8(w_fp8: np.ndarray, block_scales: np.ndarray) -> np.ndarray:
    """Exact float64 W[n, k] = E4M3(B[n, k]) * S[n // 128, k // 128]."""
    n, k = w_fp8.shape
    s = np.asarray(block_scales, dtype=np.float32).astype(np.float64)
    rows = np.arange(n) // BLOCK
    cols = np.arange(k) // BLOCK
    return E4M3[w_fp8] * s[rows][:, cols]


def linear_fp8_ref(x_bits: np.ndarray, w_fp8: np.ndarray, block_scales: np.ndarray,
                   cols: np.ndarray | None = None) -> np.ndarray:
    """y_ref[M, N] (or the selected columns) in float64."""
    x = bf16_bits_to_f64(x_bits)
    wd = dequant_fp8(w_fp8, block_scales)
    if cols is not None:
        wd = wd[cols]
    return x @ wd.T


def bound_fp8(x_bits: np.ndarray, w_fp8: np.ndarray, block_scales: np.ndarray,
              cols: np.ndarray | None = None) -> np.ndarray:
    """Sum over k of |x[m, k] * W[n, k]|, the scale of the tolerance."""
    x = np.abs(bf16_bits_to_f64(x_bits))
    wd = np.abs(dequant_fp8(w_fp8, block_scales))
    if cols is not None:
        wd = wd[cols]
    return x @ wd.T


def quantize_fp8_ref(w: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """fp32 W[N, K] (N, K multiples of 128) -> (E4M3 codes [N, K] u8,
    fp32 block scales [N/128, K/128])."""
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    if n % BLOCK or k % BLOCK:
        raise ValueError("N and K must be multiples of 128")
    w64 = w.astype(np.float64)
    if not np.all(np.isfinite(w64)):
        raise ValueError("non-finite weight")
    blocks = w64.reshape(n // BLOCK, BLOCK, k // BLOCK, BLOCK)
    amax = np.max(np.abs(blocks), axis=(1, 3))
    s = (amax / E4M3_MAX).astype(np.float32)
    s = np.where((amax == 0) | (s == 0), np.float32(1.0), s)
    v = blocks / s.astype(np.float64)[:, None, :, None]
    mag = e4m3_round(np.abs(v))
    sign = ((v < 0) & (mag != 0)).astype(np.uint8) << 7
    codes = (mag | sign).reshape(n, k).astype(np.uint8)
    return codes, s.astype(np.float32)
