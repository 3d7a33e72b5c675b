"""Python binding of libnvfp4_w4a16.so: the NVFP4 weight-only (W4A16) skinny
product on MI355X (gfx950).

Argument marshalling only: every step of the product runs in the library's HIP
kernels, every host step (packing, shape checks) in its C++.  PyTorch supplies
device memory and streams.  The C functions are declared, with their contracts,
in include/nvfp4_w4a16.h; the names here are the same without the prefix.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libnvfp4_w4a16.so")

OK = 0
ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_DTYPE, ERR_NONFINITE = -1, -2, -3, -4, -5
ERR_BADSCALE, ERR_HIP, ERR_DEVICE, ERR_TILEFILE, ERR_BUFFER = -6, -7, -8, -9, -10
ERR_TILE, ERR_SCRATCH, ERR_LIBRARY = -11, -12, -13
OUT_BF16, OUT_F32 = 0, 1
KERNEL_AUTO, KERNEL_PERSISTENT, KERNEL_TILE, KERNEL_SPLIT, KERNEL_GENERIC, KERNEL_WHOLE = 0, 1, 2, 3, 4, 5
MAX_M = 32
K_MULTIPLE = 256

EXPORTED = ("nvfp4_pack", "nvfp4_check_scales", "nvfp4_linear_shape_ok", "nvfp4_init",
            "nvfp4_linear", "nvfp4_linear_tiled", "nvfp4_tile_info", "nvfp4_strerror",
            "nvfp4_timeout_status", "nvfp4_linear_noalloc", "nvfp4_launch_info",
            "nvfp4_read_probe", "nvfp4_gemm_shape_ok", "nvfp4_gemm", "nvfp4_matmul",
            "nvfp4_dequant_bf16", "nvfp4_gemm_expanded", "nvfp4_gemm_library", "nvfp4_matmul_expand", "nvfp4_linear_dual", "nvfp4_linear_silu_input",
            "nvfp4_linear_deinterleave", "nvfp4_linear_grouped", "fp8_w8a16_pack", "fp8_w8a16_shape_ok",
            "fp8_w8a16_linear", "fp8_w8a16_gemm_shape_ok", "fp8_w8a16_gemm", "fp8_w8a16_matmul")


class Tile(ctypes.Structure):
    """nvfp4_tile_t: launch tile and kernel choice of nvfp4_linear_tiled."""
    _fields_ = [("cols", ctypes.c_int), ("waves", ctypes.c_int), ("unroll", ctypes.c_int),
                ("split", ctypes.c_int), ("mwaves", ctypes.c_int), ("kernel", ctypes.c_int)]

    def __init__(self, cols=16, waves=8, unroll=2, split=1, mwaves=0, kernel=KERNEL_AUTO):
        super().__init__(cols, waves, unroll, split, mwaves, kernel)

    def replace(self, **kw) -> "Tile":
        d = {f: getattr(self, f) for f, _ in self._fields_}
        d.update(kw)
        return Tile(**d)

    def __repr__(self) -> str:
        return "Tile(" + ", ".join(f"{f}={getattr(self, f)}" for f, _ in self._fields_) + ")"


class Nvfp4Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {strerror(status)} (status {status})")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing; build it with "
                          "`python -m verify_nvfp4_w4a16_amd.build` (no fallback exists)")
    lib = ctypes.CDLL(LIB_PATH)
    i64, vp, u8p = ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p
    lib.nvfp4_pack.argtypes = [vp, i64, i64, u8p, u8p, ctypes.POINTER(ctypes.c_float)]
    lib.nvfp4_check_scales.argtypes = [u8p, i64, i64]
    lib.nvfp4_linear_shape_ok.argtypes = [i64, i64, i64]
    lib.nvfp4_init.argtypes = []
    lib.nvfp4_linear.argtypes = [vp, vp, vp, ctypes.c_float, vp, i64, i64, i64, ctypes.c_int, vp]
    lib.nvfp4_linear_noalloc.argtypes = [vp, vp, vp, ctypes.c_float, vp, i64, i64, i64, ctypes.c_int, vp]
    lib.nvfp4_linear_tiled.argtypes = [vp, vp, vp, ctypes.c_float, vp, i64, i64, i64, ctypes.c_int,
                                       ctypes.POINTER(Tile), vp]
    lib.nvfp4_tile_info.argtypes = [i64, i64, ctypes.c_char_p, i64]
    lib.nvfp4_timeout_status.argtypes = [ctypes.POINTER(ctypes.c_int)]
    lib.nvfp4_launch_info.argtypes = [i64, i64, i64, ctypes.c_int, ctypes.c_char_p, i64]
    lib.nvfp4_read_probe.argtypes = [vp, i64, vp, i64, vp, vp]
    lib.nvfp4_gemm_shape_ok.argtypes = [i64, i64, i64]
    lib.nvfp4_gemm.argtypes = [vp, vp, vp, ctypes.c_float, vp, i64, i64, i64, ctypes.c_int, vp]
    lib.nvfp4_matmul.argtypes = [vp, vp, vp, ctypes.c_float, vp, i64, i64, i64, ctypes.c_int, vp]
    lib.nvfp4_dequant_bf16.argtypes = [vp, vp, ctypes.c_float, ctypes.c_int, vp, i64, i64, vp]
    lib.nvfp4_linear_dual.argtypes = [vp, vp, vp, ctypes.c_float, vp, vp, vp, ctypes.c_float, vp, i64, i64, i64,
                                      ctypes.c_int, vp]
    lib.nvfp4_linear_silu_input.argtypes = [vp, vp, vp, vp, ctypes.c_float, vp, i64, i64, i64, ctypes.c_int, vp]
    lib.nvfp4_linear_deinterleave.argtypes = [vp, vp, vp, ctypes.c_float, vp, i64, i64, i64, ctypes.c_int,
                                              ctypes.c_int, ctypes.POINTER(ctypes.c_int), vp]
    lib.nvfp4_linear_grouped.argtypes = [vp, i64, i64, i64, i64, ctypes.c_int, vp]
    lib.fp8_w8a16_pack.argtypes = [vp, i64, i64, vp, vp]
    lib.fp8_w8a16_shape_ok.argtypes = [i64, i64, i64]
    lib.fp8_w8a16_linear.argtypes = [vp, vp, vp, vp, i64, i64, i64, ctypes.c_int, vp]
    lib.fp8_w8a16_gemm_shape_ok.argtypes = [i64, i64, i64]
    lib.fp8_w8a16_gemm.argtypes = [vp, vp, vp, vp, i64, i64, i64, ctypes.c_int, vp]
    lib.fp8_w8a16_matmul.argtypes = [vp, vp, vp, vp, i64, i64, i64, ctypes.c_int, vp]
    lib.nvfp4_gemm_expanded.argtypes = [vp, vp, ctypes.c_float, vp, i64, i64, i64, ctypes.c_int, vp]
    lib.nvfp4_gemm_library.argtypes = [vp, vp, ctypes.c_float, vp, i64, i64, i64, ctypes.c_int, vp]
    lib.nvfp4_matmul_expand.argtypes = [vp, vp, vp, ctypes.c_float, vp, i64, i64, i64, ctypes.c_int, vp, i64, vp]
    lib.nvfp4_strerror.argtypes = [ctypes.c_int]
    lib.nvfp4_strerror.restype = ctypes.c_char_p
    for name in EXPORTED:
        if name != "nvfp4_strerror":
            getattr(lib, name).restype = ctypes.c_int
    return lib


_LIB = None


def _lib() -> ctypes.CDLL:
    """The loaded library; raises ImportError when it has not been built."""
    global _LIB
    if _LIB is None:
        _LIB = _load()
    return _LIB


def strerror(status: int) -> str:
    return _lib().nvfp4_strerror(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != OK:
        raise Nvfp4Error(status, where)


def pack(w: np.ndarray) -> tuple[np.ndarray, np.ndarray, float]:
    """fp32 W[N, K] -> (packed [N, K/2] uint8, scales [N, K/16] uint8, tensor_scale)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    if w.ndim != 2:
        raise ValueError("w must be 2-D [N, K]")
    n, k = w.shape
    packed = np.empty((n, max(k // 2, 0)), np.uint8)
    scales = np.empty((n, max(k // 16, 0)), np.uint8)
    t = ctypes.c_float()
    _check(_lib().nvfp4_pack(w.ctypes.data, n, k, packed.ctypes.data, scales.ctypes.data,
                          ctypes.byref(t)), "nvfp4_pack")
    return packed, scales, float(t.value)


def check_scales(scales: np.ndarray) -> int:
    """Status of nvfp4_check_scales for a [N, K/16] scale array (OK or ERR_BADSCALE)."""
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    return _lib().nvfp4_check_scales(scales.ctypes.data, scales.shape[0], scales.shape[1] * 16)


def linear_shape_ok(m: int, n: int, k: int) -> bool:
    return _lib().nvfp4_linear_shape_ok(m, n, k) == OK


def init() -> None:
    _check(_lib().nvfp4_init(), "nvfp4_init")


def timeout_status() -> bool:
    """True if a many-row workgroup on the current device gave up waiting for
    partial sums since the last call (waits for the device; clears the word)."""
    v = ctypes.c_int()
    _check(_lib().nvfp4_timeout_status(ctypes.byref(v)), "nvfp4_timeout_status")
    return bool(v.value)


def tile_info(n: int, k: int) -> str:
    buf = ctypes.create_string_buffer(512)
    _check(_lib().nvfp4_tile_info(n, k, buf, len(buf)), "nvfp4_tile_info")
    return buf.value.decode()


def launch_info(m: int, n: int, k: int, y_dtype: int = OUT_BF16) -> str:
    """The kernel nvfp4_linear launches for this product (trace name, grid, block, LDS)."""
    buf = ctypes.create_string_buffer(512)
    _check(_lib().nvfp4_launch_info(m, n, k, y_dtype, buf, len(buf)), "nvfp4_launch_info")
    return buf.value.decode()


def kernel_name(m: int, n: int, k: int, y_dtype: int = OUT_BF16) -> str:
    """Template name of the kernel nvfp4_linear launches, as a kernel trace shows it."""
    return launch_info(m, n, k, y_dtype).split(" grid=")[0]


def read_probe_raw(a_ptr: int, a_bytes: int, b_ptr: int, b_bytes: int, sink_ptr: int, stream: int) -> int:
    """nvfp4_read_probe on raw device addresses; returns the status."""
    return _lib().nvfp4_read_probe(a_ptr, a_bytes, b_ptr, b_bytes, sink_ptr, stream)


def table_tile(n: int, k: int) -> Tile:
    """The tile nvfp4_linear uses for an (N, K) weight (kernel left AUTO)."""
    fields = dict(kv.split("=") for kv in tile_info(n, k).split())
    return Tile(*(int(fields[f]) for f in ("cols", "waves", "unroll", "split", "mwaves")))


def linear_raw(x_ptr: int, w_ptr: int, s_ptr: int, tensor_scale: float, y_ptr: int,
               m: int, n: int, k: int, y_dtype: int, stream: int) -> int:
    """nvfp4_linear on raw device addresses; returns the status."""
    return _lib().nvfp4_linear(x_ptr, w_ptr, s_ptr, ctypes.c_float(tensor_scale), y_ptr,
                            m, n, k, y_dtype, stream)


def linear_noalloc_raw(x_ptr: int, w_ptr: int, s_ptr: int, tensor_scale: float, y_ptr: int,
                       m: int, n: int, k: int, y_dtype: int, stream: int) -> int:
    """nvfp4_linear_noalloc on raw device addresses; returns the status."""
    return _lib().nvfp4_linear_noalloc(x_ptr, w_ptr, s_ptr, ctypes.c_float(tensor_scale), y_ptr,
                                       m, n, k, y_dtype, stream)


def gemm_raw(x_ptr: int, w_ptr: int, s_ptr: int, tensor_scale: float, y_ptr: int,
             m: int, n: int, k: int, y_dtype: int, stream: int) -> int:
    """nvfp4_gemm on raw device addresses; returns the status."""
    return _lib().nvfp4_gemm(x_ptr, w_ptr, s_ptr, ctypes.c_float(tensor_scale), y_ptr, m, n, k, y_dtype, stream)


def matmul_raw(x_ptr: int, w_ptr: int, s_ptr: int, tensor_scale: float, y_ptr: int,
               m: int, n: int, k: int, y_dtype: int, stream: int) -> int:
    """nvfp4_matmul on raw device addresses; returns the status."""
    return _lib().nvfp4_matmul(x_ptr, w_ptr, s_ptr, ctypes.c_float(tensor_scale), y_ptr, m, n, k, y_dtype, stream)


def dequant_bf16_raw(w_ptr: int, s_ptr: int, tensor_scale: float, apply_tensor_scale: int, dst_ptr: int,
                     n: int, k: int, stream: int) -> int:
    """nvfp4_dequant_bf16 on raw device addresses; returns the status."""
    return _lib().nvfp4_dequant_bf16(w_ptr, s_ptr, ctypes.c_float(tensor_scale), apply_tensor_scale, dst_ptr,
                                     n, k, stream)


def gemm_expanded_raw(x_ptr: int, wbf_ptr: int, tensor_scale: float, y_ptr: int,
                      m: int, n: int, k: int, y_dtype: int, stream: int) -> int:
    """nvfp4_gemm_expanded on raw device addresses; returns the status."""
    return _lib().nvfp4_gemm_expanded(x_ptr, wbf_ptr, ctypes.c_float(tensor_scale), y_ptr, m, n, k, y_dtype,
                                      stream)


def gemm_library_raw(x_ptr: int, wbf_ptr: int, tensor_scale: float, y_ptr: int,
                     m: int, n: int, k: int, y_dtype: int, stream: int) -> int:
    """nvfp4_gemm_library on raw device addresses; returns the status."""
    return _lib().nvfp4_gemm_library(x_ptr, wbf_ptr, ctypes.c_float(tensor_scale), y_ptr, m, n, k, y_dtype,
                                     stream)


def matmul_expand_raw(x_ptr: int, w_ptr: int, s_ptr: int, tensor_scale: float, y_ptr: int, m: int, n: int, k: int,
                      y_dtype: int, scratch_ptr: int, expand_min_m: int, stream: int) -> int:
    """nvfp4_matmul_expand on raw device addresses; returns the status."""
    return _lib().nvfp4_matmul_expand(x_ptr, w_ptr, s_ptr, ctypes.c_float(tensor_scale), y_ptr, m, n, k, y_dtype,
                                      scratch_ptr, expand_min_m, stream)


def linear_dual_raw(x_ptr, w0_ptr, s0_ptr, t0, y0_ptr, w1_ptr, s1_ptr, t1, y1_ptr, m, n, k, y_dtype,
                    stream) -> int:
    """nvfp4_linear_dual on raw device addresses; returns the status."""
    return _lib().nvfp4_linear_dual(x_ptr, w0_ptr, s0_ptr, ctypes.c_float(t0), y0_ptr, w1_ptr, s1_ptr,
                                    ctypes.c_float(t1), y1_ptr, m, n, k, y_dtype, stream)


def linear_silu_input_raw(gate_ptr, up_ptr, w_ptr, s_ptr, tensor_scale, y_ptr, m, n, k, y_dtype,
                          stream) -> int:
    """nvfp4_linear_silu_input on raw device addresses; returns the status."""
    return _lib().nvfp4_linear_silu_input(gate_ptr, up_ptr, w_ptr, s_ptr, ctypes.c_float(tensor_scale), y_ptr,
                                          m, n, k, y_dtype, stream)


def linear_deinterleave_raw(x_ptr, w_ptr, s_ptr, tensor_scale, y_ptr, m, n, k, y_dtype, widths,
                            stream) -> int:
    """nvfp4_linear_deinterleave on raw device addresses; `widths` a list of part widths."""
    arr = (ctypes.c_int * len(widths))(*widths) if widths is not None else None
    return _lib().nvfp4_linear_deinterleave(x_ptr, w_ptr, s_ptr, ctypes.c_float(tensor_scale), y_ptr, m, n, k,
                                            y_dtype, len(widths) if widths is not None else 0, arr, stream)


# nvfp4_group_t: four device pointers, the fp32 tensor scale, the int32 row count
GROUP_DTYPE = np.dtype([("x", "<u8"), ("w_packed", "<u8"), ("scales_e4m3", "<u8"), ("y", "<u8"),
                        ("tensor_scale", "<f4"), ("m", "<i4")])


def linear_grouped_raw(table_ptr, count, max_m, n, k, y_dtype, stream) -> int:
    """nvfp4_linear_grouped on a device table of GROUP_DTYPE records; returns the status."""
    return _lib().nvfp4_linear_grouped(table_ptr, count, max_m, n, k, y_dtype, stream)


def fp8_pack(w: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """fp32 W[N, K] -> (e4m3 codes [N, K] uint8, fp32 block scales [N/128, K/128])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    if w.ndim != 2:
        raise ValueError("w must be 2-D [N, K]")
    n, k = w.shape
    codes = np.empty((n, k), np.uint8)
    scales = np.empty((max(n // 128, 0), max(k // 128, 0)), np.float32)
    _check(_lib().fp8_w8a16_pack(w.ctypes.data, n, k, codes.ctypes.data, scales.ctypes.data), "fp8_w8a16_pack")
    return codes, scales


def fp8_shape_ok(m: int, n: int, k: int) -> bool:
    return _lib().fp8_w8a16_shape_ok(m, n, k) == OK


def fp8_linear_raw(x_ptr, w_ptr, s_ptr, y_ptr, m, n, k, y_dtype, stream) -> int:
    """fp8_w8a16_linear on raw device addresses; returns the status."""
    return _lib().fp8_w8a16_linear(x_ptr, w_ptr, s_ptr, y_ptr, m, n, k, y_dtype, stream)


def fp8_gemm_shape_ok(m: int, n: int, k: int) -> bool:
    return _lib().fp8_w8a16_gemm_shape_ok(m, n, k) == OK


def fp8_gemm_raw(x_ptr, w_ptr, s_ptr, y_ptr, m, n, k, y_dtype, stream) -> int:
    """fp8_w8a16_gemm on raw device addresses; returns the status."""
    return _lib().fp8_w8a16_gemm(x_ptr, w_ptr, s_ptr, y_ptr, m, n, k, y_dtype, stream)


def fp8_matmul_raw(x_ptr, w_ptr, s_ptr, y_ptr, m, n, k, y_dtype, stream) -> int:
    """fp8_w8a16_matmul on raw device addresses; returns the status."""
    return _lib().fp8_w8a16_matmul(x_ptr, w_ptr, s_ptr, y_ptr, m, n, k, y_dtype, stream)


def gemm_shape_ok(m: int, n: int, k: int) -> bool:
    return _lib().nvfp4_gemm_shape_ok(m, n, k) == OK


def linear_tiled_raw(x_ptr: int, w_ptr: int, s_ptr: int, tensor_scale: float, y_ptr: int,
                     m: int, n: int, k: int, y_dtype: int, tile: Tile | None, stream: int) -> int:
    """nvfp4_linear_tiled on raw device addresses; returns the status."""
    ref = ctypes.byref(tile) if tile is not None else None
    return _lib().nvfp4_linear_tiled(x_ptr, w_ptr, s_ptr, ctypes.c_float(tensor_scale), y_ptr,
                                     m, n, k, y_dtype, ref, stream)


def linear(x, w_packed, scales, tensor_scale: float, out=None, out_dtype=None, stream=None,
           tile=None):
    """y[M, N] = x[M, K] . dequant(W)^T on the GPU (torch tensors on one device).

    x: bf16 [M, K]; w_packed: uint8 [N, K/2]; scales: uint8 [N, K/16];
    out: bf16 or float32 [M, N] (allocated when None; dtype from out_dtype,
    default bf16).  Runs on `stream` (default: torch's current stream).  `tile`
    (a Tile) selects nvfp4_linear_tiled with that launch tile and kernel."""
    import torch
    if x.dtype != torch.bfloat16 or w_packed.dtype != torch.uint8 or scales.dtype != torch.uint8:
        raise TypeError("x must be bfloat16; w_packed and scales uint8")
    if x.dim() != 2 or w_packed.dim() != 2 or scales.dim() != 2:
        raise ValueError("x, w_packed, scales must be 2-D")
    m, k = x.shape
    n = w_packed.shape[0]
    if tuple(w_packed.shape) != (n, k // 2) or tuple(scales.shape) != (n, k // 16):
        raise ValueError(f"weight shapes {tuple(w_packed.shape)}, {tuple(scales.shape)} "
                         f"do not match K={k}")
    for name, tns in (("x", x), ("w_packed", w_packed), ("scales", scales)):
        if not tns.is_cuda or not tns.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype or torch.bfloat16, device=x.device)
    if out.dtype not in (torch.bfloat16, torch.float32) or tuple(out.shape) != (m, n) \
            or not out.is_contiguous() or out.device != x.device:
        raise ValueError("out must be a contiguous bf16 or float32 [M, N] tensor on x's device")
    y_dtype = OUT_F32 if out.dtype == torch.float32 else OUT_BF16
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    if tile is None:
        st = linear_raw(x.data_ptr(), w_packed.data_ptr(), scales.data_ptr(), tensor_scale,
                        out.data_ptr(), m, n, k, y_dtype, stream.cuda_stream)
    else:
        if not isinstance(tile, Tile):
            raise TypeError("tile must be a Tile")
        st = linear_tiled_raw(x.data_ptr(), w_packed.data_ptr(), scales.data_ptr(), tensor_scale,
                              out.data_ptr(), m, n, k, y_dtype, tile, stream.cuda_stream)
    _check(st, "nvfp4_linear" if tile is None else "nvfp4_linear_tiled")
    return out
