"""The NVFP4 W4A16 product in float64, and its acceptance test.

y[m, n] = sum_k x[m, k] * Wd[n, k], with
Wd[n, k] = t * E4M3(scales[n, k // 16]) * E2M1(q[n, k]) and
q[n, k] = nibble (k mod 2) of byte w_packed[n, k // 2], the low nibble for even k.

Sources ("Module ops", metrale_model_layers::layers::ops):
``w4a16_gemm`` and ``w4a16_gemv`` give C = A @ dequant(B) with A bf16 [M, K];
``w4a16_tc_rows`` gives output = input x W^T for the row-major NVFP4 weight
[n, k] with e4m3 scales of 16; ``dequant_nvfp4_to_bf16`` multiplies by the
per-tensor scale; ``nvfp4_mmq_repack`` fixes packed [n, k/2] with the low nibble
holding the even k and the scales as [n, k/16].

Every product t * e4m3 * e2m1 has at most 24 + 4 + 2 significant bits, so
``dequant`` is exact in float64; ``linear_ref`` then adds K exact products in
float64 through a BLAS dgemm.
"""
from __future__ import annotations

import numpy as np

from .formats import E2M1, E4M3

GROUP = 16          # k per e4m3 scale
ROW_BLOCK = 4096    # rows of W decoded at a time, to bound memory


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact float64 value of each bf16 (given as uint16 bit patterns)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def nibble_shift(k: np.ndarray) -> np.ndarray:
    """Bit offset of element k inside its byte: the low nibble holds even k."""
    return 4 * (k % 2)


def scale_index(k: np.ndarray) -> np.ndarray:
    """Scale byte of element k inside its row: 16 consecutive k share one."""
    return k // GROUP


def unpack_codes(w_packed: np.ndarray, k: int) -> np.ndarray:
    """[n, k/2] bytes -> [n, k] e2m1 codes."""
    ks = np.arange(k)
    bytes_ = w_packed[:, ks // 2].astype(np.uint8)
    return (bytes_ >> nibble_shift(ks).astype(np.uint8)) & 0xF


def dequant(w_packed: np.ndarray, scales: np.ndarray, t: float,
            rows: slice | None = None) -> np.ndarray:
    """Exact float64 Wd[n, k] for the selected rows."""
    if rows is not None:
        w_packed, scales = w_packed[rows], scales[rows]
    k = w_packed.shape[1] * 2
    codes = unpack_codes(w_packed, k)
    group_scale = E4M3[scales[:, scale_index(np.arange(k))]]
    return np.float64(np.float32(t)) * group_scale * E2M1[codes]


def linear_ref(x_bits: np.ndarray, w_packed: np.ndarray, scales: np.ndarray,
               t: float, cols: np.ndarray | None = None) -> np.ndarray:
    """y_ref[M, N] (or [M, len(cols)]) = x @ Wd^T in float64."""
    x = bf16_bits_to_f64(x_bits)
    if cols is not None:
        wd = dequant(w_packed[cols], scales[cols], t)
        return x @ wd.T
    n = w_packed.shape[0]
    out = np.empty((x.shape[0], n), dtype=np.float64)
    for r0 in range(0, n, ROW_BLOCK):
        r = slice(r0, min(n, r0 + ROW_BLOCK))
        out[:, r] = x @ dequant(w_packed, scales, t, r).T
    return out


def bound(x_bits: np.ndarray, w_packed: np.ndarray, scales: np.ndarray,
          t: float, cols: np.ndarray | None = None) -> np.ndarray:
    """Sum over k of |x[m, k] * Wd[n, k]|, the scale of the tolerance."""
    x = np.abs(bf16_bits_to_f64(x_bits))
    if cols is not None:
        return x @ np.abs(dequant(w_packed[cols], scales[cols], t)).T
    n = w_packed.shape[0]
    out = np.empty((x.shape[0], n), dtype=np.float64)
    for r0 in range(0, n, ROW_BLOCK):
        r = slice(r0, min(n, r0 + ROW_BLOCK))
        out[:, r] = x @ np.abs(dequant(w_packed, scales, t, r)).T
    return out


REL_TOL = 2e-3
ABS_TOL = 1e-6
# bf16 keeps 8 significant bits, so rounding a value to the nearest bf16 moves
# it by up to 2^-8 of itself.
BF16_UNIT_ROUNDOFF = 2.0 ** -8


def tolerance(y_ref: np.ndarray, bnd: np.ndarray, out: str = "f32") -> np.ndarray:
    """Allowed |y - y_ref| per element: 2e-3 * bound + 1e-6 for the product.

    A bf16 output carries one more rounding, of at most 2^-8 of the value;
    the 2e-3 term alone cannot hold it when a single product dominates the sum
    ("CUDA Kernel Engineering", "Writing a new kernel", compares BF16 outputs
    with a relative allowance of 1e-2 for the same reason), so for out="bf16"
    that rounding is added on top."""
    tol = REL_TOL * bnd + ABS_TOL
    if out == "bf16":
        tol = tol + BF16_UNIT_ROUNDOFF * (np.abs(y_ref) + tol)
    elif out != "f32":
        raise ValueError("out must be 'f32' or 'bf16'")
    return tol


def max_violation(y: np.ndarray, y_ref: np.ndarray, bnd: np.ndarray, out: str = "f32") -> float:
    """max over elements of |y - y_ref| / tolerance; <= 1 means accepted.

    A NaN in y counts as a violation unless y_ref is NaN at the same place."""
    y = np.asarray(y, dtype=np.float64)
    err = np.abs(y - y_ref) / tolerance(y_ref, bnd, out)
    both_nan = np.isnan(y) & np.isnan(y_ref)
    err = np.where(both_nan, 0.0, err)
    err = np.where(np.isnan(err), np.inf, err)
    return float(err.max()) if err.size else 0.0


def accept(y: np.ndarray, y_ref: np.ndarray, bnd: np.ndarray, out: str = "f32") -> bool:
    """Element-wise |y - y_ref| <= tolerance(y_ref, bound, out)."""
    return max_violation(y, y_ref, bnd, out) <= 1.0
