"""The FP8 block-scaled product (W8A16) on the GPU (gpu): parity with the fp64
oracle, exact decode of every e4m3 code, and each row's bits independent of M
and of the other rows."""
import numpy as np
import pytest
import torch

import oracle
import verify_nvfp4_w4a16_amd as nv
import workload
from tests._gpu import DEV, bits, to_f64, upload_bits, upload_u8

pytestmark = pytest.mark.gpu


def _run(xd, wd, sd, m, n, k, out_dtype=torch.bfloat16):
    y = torch.empty((m, n), dtype=out_dtype, device=DEV)
    od = nv.OUT_F32 if out_dtype == torch.float32 else nv.OUT_BF16
    st = nv.fp8_linear_raw(xd.data_ptr(), wd.data_ptr(), sd.data_ptr(), y.data_ptr(), m, n, k, od,
                           torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == nv.OK, st
    return y


def _parity(y, x, codes, scales, cols=None, label=""):
    y64 = to_f64(y)
    if cols is not None:
        y64 = y64[:, cols]
    ref = oracle.linear_fp8_ref(x, codes, scales, cols)
    bnd = oracle.bound_fp8(x, codes, scales, cols)
    out = "bf16" if y.dtype == torch.bfloat16 else "f32"
    viol = oracle.max_violation(y64, ref, bnd, out)
    print(f"[parity] {label} {out} M={x.shape[0]} max err/tol = {viol:.3g}", flush=True)
    assert viol <= 1.0, label


def test_w8a16_parity_and_row_invariance():
    # (column tiles per wavefront: 1 where x fits the LDS, else 2 from 8192
    # columns, so the row comparisons below cross them)
    for n, k in [(4096, 4096), (8192, 4096), (4096, 12288), (384, 1152), (16384, 2048)]:
        codes, scales = nv.fp8_pack(workload.weights_f32(n, k, 100 + n // 128))
        wd, sd = upload_u8(codes), torch.from_numpy(scales).to(DEV)
        x = workload.activations_bf16(32, k, 200 + k, outliers=True)
        xd = upload_bits(x)
        full = _run(xd, wd, sd, 32, n, k)
        cols = np.unique(np.concatenate([np.arange(32), np.arange(n - 32, n),
                                         workload.rng(n).integers(0, n, 256)]))
        _parity(full, x, codes, scales, cols, f"w8a16 {n}x{k} M=32")
        ref = bits(full).clone()
        for m in (1, 2, 5, 7, 8, 16, 17, 31):
            y = _run(xd, wd, sd, m, n, k)
            assert torch.equal(bits(y), ref[:m]), (n, k, m)     # x in LDS (small M) or read per chunk
        alone = _run(upload_bits(x[9:10]), wd, sd, 1, n, k)
        assert torch.equal(bits(alone), ref[9:10])
        _parity(_run(xd, wd, sd, 3, n, k, torch.float32), x[:3], codes, scales, cols, f"w8a16 {n}x{k} fp32")


def test_w8a16_every_code_decoded_exactly():
    # One-hot x picks single weights: y[m, n] = e4m3(code) * S exactly, for
    # all 256 codes (0x7F and 0xFF give NaN) at two scales.
    n, k = 256, 256
    codes = np.zeros((n, k), np.uint8)
    codes[:, 3] = np.arange(256, dtype=np.uint8)
    scales = np.array([[2.0 ** -3, 1.0], [3.0, 0.5]], np.float32)
    x = np.zeros((1, k), np.uint16)
    x[0, 3] = 0x3F80
    y = _run(upload_bits(x), upload_u8(codes), torch.from_numpy(scales).to(DEV), 1, n, k, torch.float32)
    got = y.cpu().numpy()[0].astype(np.float64)
    want = oracle.E4M3[np.arange(256)] * np.where(np.arange(256) < 128, 2.0 ** -3, 3.0)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])


def test_w8a16_errors():
    codes, scales = nv.fp8_pack(workload.weights_f32(128, 256, 5))
    wd, sd = upload_u8(codes), torch.from_numpy(scales).to(DEV)
    x = upload_bits(workload.activations_bf16(2, 256, 6))
    y = torch.empty((2, 128), dtype=torch.bfloat16, device=DEV)
    s = torch.cuda.current_stream().cuda_stream
    assert nv.fp8_linear_raw(x.data_ptr(), wd.data_ptr(), sd.data_ptr(), y.data_ptr(), 33, 128, 256, 0, s) == \
        nv.ERR_SHAPE
    assert nv.fp8_linear_raw(x.data_ptr(), wd.data_ptr(), sd.data_ptr(), y.data_ptr(), 2, 100, 256, 0, s) == \
        nv.ERR_SHAPE
    assert nv.fp8_linear_raw(x.data_ptr() + 8, wd.data_ptr(), sd.data_ptr(), y.data_ptr(), 2, 128, 256, 0, s) == \
        nv.ERR_ALIGN
    assert nv.fp8_linear_raw(x.data_ptr(), wd.data_ptr(), sd.data_ptr(), y.data_ptr(), 0, 128, 256, 0, s) == nv.OK


def _gemm(xd, wd, sd, m, n, k, out_dtype=torch.bfloat16, fn=None):
    y = torch.empty((m, n), dtype=out_dtype, device=DEV)
    od = nv.OUT_F32 if out_dtype == torch.float32 else nv.OUT_BF16
    st = (fn or nv.fp8_gemm_raw)(xd.data_ptr(), wd.data_ptr(), sd.data_ptr(), y.data_ptr(), m, n, k, od,
                                 torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == nv.OK, st
    return y


def test_w8a16_gemm_rows_equal_linear_rows_and_parity():
    # Many rows: every row has the bits fp8_w8a16_linear gives it (32-row
    # slices and a single row), at every M, with and without the K split
    # (4096 columns at 256 rows split; 1024 rows do not), ragged M; parity on
    # sampled columns.
    for n, k in [(4096, 4096), (8192, 4096), (4096, 12288), (384, 1152)]:
        codes, scales = nv.fp8_pack(workload.weights_f32(n, k, 300 + n // 128))
        wd, sd = upload_u8(codes), torch.from_numpy(scales).to(DEV)
        x = workload.activations_bf16(1024, k, 400 + k, outliers=True)
        xd = upload_bits(x)
        full = bits(_gemm(xd, wd, sd, 1024, n, k)).clone()
        for r0 in (0, 32, 992):
            lin = bits(_run(upload_bits(x[r0:r0 + 32]), wd, sd, 32, n, k))
            assert torch.equal(lin, full[r0:r0 + 32]), (n, k, r0)
        assert torch.equal(bits(_run(upload_bits(x[77:78]), wd, sd, 1, n, k)), full[77:78])
        for m in (33, 70, 256, 600):
            y = _gemm(xd, wd, sd, m, n, k)
            assert torch.equal(bits(y), full[:m]), (n, k, m)
            y = _gemm(xd, wd, sd, m, n, k, fn=nv.fp8_matmul_raw)
            assert torch.equal(bits(y), full[:m]), (n, k, m, "matmul")
        cols = np.unique(np.concatenate([np.arange(16), np.arange(n - 16, n), workload.rng(n + 1).integers(0, n, 96)]))
        _parity(_gemm(xd, wd, sd, 1024, n, k), x, codes, scales, cols, f"w8a16 gemm {n}x{k}")
        _parity(_gemm(xd, wd, sd, 70, n, k, torch.float32), x[:70], codes, scales, cols, f"w8a16 gemm {n}x{k} fp32")


def test_w8a16_many_row_form_fp32_and_ragged_groups():
    # The many-row form at each of its dispatches, fp32 and bf16 output:
    # 4096 columns (segment groups meeting through the exchange), 8192
    # (whole K, two wavefronts), 24704 (whole K, six wavefronts, the last
    # workgroup's columns past N); rows equal the FP8 GEMM's, parity on
    # sampled columns including the last ones.
    for n, k, ms in [(4096, 4096, (9, 16, 32)), (8192, 4096, (16, 17)), (24704, 4096, (16,))]:
        codes, scales = nv.fp8_pack(workload.weights_f32(n, k, 500 + n // 128))
        wd, sd = upload_u8(codes), torch.from_numpy(scales).to(DEV)
        x = workload.activations_bf16(32, k, 600 + n // 128, outliers=True)
        cols = np.unique(np.concatenate([np.arange(16), np.arange(n - 48, n), workload.rng(n + 2).integers(0, n, 64)]))
        for m in ms:
            xd = upload_bits(x[:m])
            for out in (torch.float32, torch.bfloat16):
                y = _run(xd, wd, sd, m, n, k, out)
                assert torch.equal(bits(y), bits(_gemm(xd, wd, sd, m, n, k, out))), (n, k, m, out)
                _parity(y, x[:m], codes, scales, cols, f"w8a16 many-row {n}x{k}")


def test_w8a16_gemm_contract_and_errors():
    assert nv.fp8_gemm_shape_ok(0, 128, 128) and nv.fp8_gemm_shape_ok(4096, 8192, 4096)
    assert not nv.fp8_gemm_shape_ok(64, 100, 128) and not nv.fp8_gemm_shape_ok(64, 128, 100)
    assert not nv.fp8_gemm_shape_ok(-1, 128, 128)
    codes, scales = nv.fp8_pack(workload.weights_f32(128, 256, 5))
    wd, sd = upload_u8(codes), torch.from_numpy(scales).to(DEV)
    x = torch.zeros((40, 256), dtype=torch.bfloat16, device=DEV)
    y = torch.empty((40, 128), dtype=torch.bfloat16, device=DEV)
    s = torch.cuda.current_stream().cuda_stream
    assert nv.fp8_gemm_raw(x.data_ptr(), wd.data_ptr(), sd.data_ptr(), y.data_ptr(), 0, 128, 256, 0, s) == nv.OK
    assert nv.fp8_gemm_raw(x.data_ptr() + 2, wd.data_ptr(), sd.data_ptr(), y.data_ptr(), 40, 128, 256, 0, s) == \
        nv.ERR_ALIGN
    assert nv.fp8_gemm_raw(x.data_ptr(), wd.data_ptr(), sd.data_ptr(), y.data_ptr(), 40, 128, 256, 5, s) == \
        nv.ERR_DTYPE
    assert nv.fp8_gemm_raw(x.data_ptr(), 0, sd.data_ptr(), y.data_ptr(), 40, 128, 256, 0, s) == nv.ERR_NULL
    assert nv.fp8_matmul_raw(x.data_ptr(), wd.data_ptr(), sd.data_ptr(), y.data_ptr(), 40, 128, 200, 0, s) == \
        nv.ERR_SHAPE
