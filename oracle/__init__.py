"""Oracle for the NVFP4 weight-only product (W4A16): TEST INFRASTRUCTURE ONLY.

A plain, slow CPU implementation in float64 of what the HIP library computes,
written from the pages' description of the NVFP4 format and product:

* "10 Kernels", section 10.2 (NVFP4 matrix products): 4-bit e2m1 weights with
  an e4m3 scale per group, 16-bit activations, and the fact that an e2m1 value
  times an e4m3 scale is exact in fp16;
* "Module ops" (metrale_model_layers::layers::ops): ``w4a16_gemm`` /
  ``w4a16_gemv`` (C = A @ dequant(B), A [M,K] bf16, B NVFP4 = packed e2m1,
  e4m3 block scales, fp32 per-tensor scale), ``w4a16_tc_rows`` (row-major
  NVFP4 weight [n,k], e4m3 scales of 16), ``dequant_nvfp4_to_bf16`` (the
  per-tensor scale multiplies the dequantised weight), ``nvfp4_mmq_repack``
  (packed e2m1 [n,k/2] with the low nibble holding the even k; e4m3 [n,k/16]),
  ``quantize_bf16_to_nvfp4`` and the constant ``E4M3_MAX``.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP path and
the product never calls it.

Every function here is pinned by a ``-m "not gpu"`` test to something other
than itself (published format definitions, library routines, exact rational
arithmetic, closed forms).  No function is "parity unpinned".
"""
from .formats import E2M1, E4M3, e2m1_value, e4m3_value
from .linear import (unpack_codes, dequant, linear_ref, bound, accept,
                     max_violation, tolerance, bf16_bits_to_f64)
from .quant import quantize_ref, e4m3_round, e2m1_round
from .expand import round_to_bf16, dequant_bf16
from .fused import silu, silu_mul_bf16, deinterleave_columns, deinterleave
from .fp8 import dequant_fp8, linear_fp8_ref, bound_fp8, quantize_fp8_ref

__all__ = ["E2M1", "E4M3", "e2m1_value", "e4m3_value", "unpack_codes",
           "dequant", "linear_ref", "bound", "accept", "max_violation", "tolerance",
           "bf16_bits_to_f64", "quantize_ref", "e4m3_round", "e2m1_round", "round_to_bf16",
           "dequant_bf16", "silu", "silu_mul_bf16", "deinterleave_columns", "deinterleave",
           "dequant_fp8", "linear_fp8_ref", "bound_fp8", "quantize_fp8_ref"]
