"""Helpers shared by the GPU tests: uploads, one product through the C ABI,
and the oracle comparison.  Not a test module."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import verify_nvfp4_w4a16_amd as nv

DEV = torch.device("cuda:0")


def upload_bits(xb: np.ndarray) -> torch.Tensor:
    """bf16 bit patterns (uint16 numpy) -> bf16 tensor on the GPU."""
    return torch.from_numpy(np.ascontiguousarray(xb).view(np.int16)).to(DEV).view(torch.bfloat16)


def upload_u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


class Weight:
    """A packed weight kept on the host (for the oracle) and on the GPU."""

    def __init__(self, packed: np.ndarray, scales: np.ndarray, t: float):
        self.packed, self.scales, self.t = packed, scales, float(t)
        self.n, self.k = packed.shape[0], packed.shape[1] * 2
        self.wp = upload_u8(packed)
        self.sc = upload_u8(scales)

    @classmethod
    def from_f32(cls, w: np.ndarray) -> "Weight":
        return cls(*nv.pack(w))


def run(x_bits: np.ndarray, w: Weight, out_dtype=torch.bfloat16) -> torch.Tensor:
    y = nv.linear(upload_bits(x_bits), w.wp, w.sc, w.t, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return y


def to_f64(y: torch.Tensor) -> np.ndarray:
    return y.float().cpu().numpy().astype(np.float64)


def check_parity(y: torch.Tensor, x_bits: np.ndarray, w: Weight, cols=None, label=""):
    """Element-wise |y - y_ref| <= 2e-3 * bound + 1e-6 against the fp64 oracle."""
    y64 = to_f64(y)
    if cols is not None:
        y64 = y64[:, cols]
    y_ref = oracle.linear_ref(x_bits, w.packed, w.scales, w.t, cols)
    bnd = oracle.bound(x_bits, w.packed, w.scales, w.t, cols)
    out = "bf16" if y.dtype == torch.bfloat16 else "f32"
    viol = oracle.max_violation(y64, y_ref, bnd, out)
    print(f"[parity] {label} {out} M={x_bits.shape[0]} N={w.n} K={w.k} max err/tol = {viol:.3g}", flush=True)
    assert viol <= 1.0, f"{label}: tolerance exceeded, max err/tol = {viol}"
    return viol


def bits(y: torch.Tensor) -> torch.Tensor:
    return y.view(torch.int16) if y.dtype == torch.bfloat16 else y.view(torch.int32)
