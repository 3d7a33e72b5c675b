"""The many-row regime (nvfp4_gemm), the expand-to-bf16 regime
(nvfp4_dequant_bf16 + nvfp4_gemm_expanded, or + nvfp4_gemm_library) and the
row-count dispatcher (nvfp4_matmul) on the GPU: parity with the fp64 oracle,
bit-exact expansion, and every row's bits equal to nvfp4_linear's for the
same row, except on the library GEMM, which picks its own K order (gpu)."""
import numpy as np
import pytest
import torch

import oracle
import verify_nvfp4_w4a16_amd as nv
import workload
from tests._gpu import DEV, Weight, bits, check_parity, upload_bits

pytestmark = pytest.mark.gpu


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _gemm(xd, w, m, out_dtype=torch.bfloat16, fn=None):
    y = torch.empty((m, w.n), dtype=out_dtype, device=DEV)
    od = nv.OUT_F32 if out_dtype == torch.float32 else nv.OUT_BF16
    st = (fn or nv.gemm_raw)(xd.data_ptr(), w.wp.data_ptr(), w.sc.data_ptr(), w.t, y.data_ptr(), m, w.n, w.k,
                             od, _stream())
    torch.cuda.synchronize()
    assert st == nv.OK, st
    return y


def _linear(xd, w, m, out_dtype=torch.bfloat16):
    y = torch.empty((m, w.n), dtype=out_dtype, device=DEV)
    od = nv.OUT_F32 if out_dtype == torch.float32 else nv.OUT_BF16
    st = nv.linear_raw(xd.data_ptr(), w.wp.data_ptr(), w.sc.data_ptr(), w.t, y.data_ptr(), m, w.n, w.k, od,
                       _stream())
    torch.cuda.synchronize()
    assert st == nv.OK, st
    return y


def _expanded(w, apply_t):
    dst = torch.empty((w.n, w.k), dtype=torch.int16, device=DEV)
    st = nv.dequant_bf16_raw(w.wp.data_ptr(), w.sc.data_ptr(), w.t, 1 if apply_t else 0, dst.data_ptr(),
                             w.n, w.k, _stream())
    torch.cuda.synchronize()
    assert st == nv.OK, st
    return dst


@pytest.mark.parametrize("shape", workload.ROUND_SHAPES, ids=lambda s: f"{s.n}x{s.k}")
def test_gemm_parity_and_rows_across_m(shape):
    # The decode round's shapes at 33, 64, 256 and 1024 rows (the regime's
    # span): within the oracle's tolerance on sampled columns, and each row's
    # bits the same at every M (the first rows of the 1024-row product).
    w = Weight.from_f32(workload.weights_f32(shape.n, shape.k, workload.round_weight_seed(0, 0) + shape.n))
    x = workload.activations_bf16(1024, shape.k, 7000 + shape.k)
    xd = upload_bits(x)
    cols = np.unique(np.concatenate([np.arange(16), np.arange(shape.n - 16, shape.n),
                                     workload.rng(71).integers(0, shape.n, 96)]))
    full = bits(_gemm(xd, w, 1024)).clone()
    assert torch.equal(bits(_gemm(xd, w, 1024, fn=nv.matmul_raw)), full)
    assert torch.equal(bits(_gemm(xd, w, 100, fn=nv.matmul_raw)), full[:100])
    rows = np.unique(np.concatenate([np.arange(8), workload.rng(72).integers(0, 1024, 56)]))
    check_parity(_gemm(xd, w, 1024)[torch.from_numpy(rows).to(DEV)], x[rows], w, cols=cols,
                 label=f"gemm {shape.n}x{shape.k} M=1024 sampled rows")
    for m in (33, 64, 256):
        y = _gemm(xd, w, m)
        assert torch.equal(bits(y), full[:m]), f"{shape.n}x{shape.k}: rows at M={m} differ from M=1024"
        if m == 33:
            check_parity(y, x[:m], w, cols=cols, label=f"gemm {shape.n}x{shape.k} M={m}")


def test_gemm_rows_equal_linear_rows():
    # The same row gets the same bits from nvfp4_gemm at any M and from
    # nvfp4_linear at 1..32 rows (one K order for both), on the row-count
    # dispatcher's boundary too (32 -> linear, 33 -> gemm).
    n, k = 4136, 4096                              # ragged columns for both kernels' tiles
    w = Weight.from_f32(workload.weights_f32(n, k, 81))
    x = workload.activations_bf16(96, k, 82)
    xd = upload_bits(x)
    g = bits(_gemm(xd, w, 96)).clone()
    for r0 in (0, 32, 64):
        lin = bits(_linear(upload_bits(x[r0:r0 + 32]), w, 32))
        assert torch.equal(lin, g[r0:r0 + 32]), r0
    assert torch.equal(bits(_linear(upload_bits(x[5:6]), w, 1)), g[5:6])
    for m in (32, 33, 64, 65, 96):
        y = _gemm(xd, w, m, fn=nv.matmul_raw)                # 32-row slices in one launch up to 64 rows, then the GEMM
        assert torch.equal(bits(y), g[:m]), m
    check_parity(_gemm(xd, w, 96, torch.float32), x, w, label="gemm 4136x4096 M=96 fp32")


def test_gemm_k_split_rows_equal_unsplit():
    # No more 128 x 64 tiles than CUs: each workgroup takes one segment group
    # and a second kernel adds the group sums in order.  Every row's bits
    # equal those of a product with enough rows to run unsplit (bf16 and fp32
    # outputs, ragged columns), and the split product is within the oracle's
    # tolerance.
    for n, k in [(4096, 8192), (4100, 4096)]:
        w = Weight.from_f32(workload.weights_f32(n, k, n + 5))
        x = workload.activations_bf16(1536, k, k + 6)
        xd = upload_bits(x)
        for dt in (torch.bfloat16, torch.float32):
            full = bits(_gemm(xd, w, 1536, dt)).clone()
            for m in (1, 40, 200, 255):
                assert torch.equal(bits(_gemm(xd, w, m, dt)), full[:m]), (n, k, m, dt)
        cols = np.unique(np.concatenate([np.arange(8), np.arange(n - 8, n), workload.rng(n).integers(0, n, 48)]))
        check_parity(_gemm(xd, w, 200, torch.float32), x[:200], w, cols=cols, label=f"k-split gemm {n}x{k} M=200")


def test_gemm_ragged_rows_random_codes():
    # Partial row tiles (M = 200, 129, 1), columns past N, every code and
    # scale byte incl. subnormal scales and zero groups, split shapes.
    # (24704 columns at 200 rows: 64-row tiles, ragged in rows and columns)
    for n, k, m in [(333, 1024, 200), (4111, 512, 129), (17, 256, 1), (1000, 2048, 300), (24704, 1024, 200)]:
        packed, scales = workload.random_codes(n, k, n + k)
        scales[:, ::5] = 0
        w = Weight(packed, scales, 0.0371)
        x = workload.activations_bf16(m, k, n * 3 + m, outliers=True)
        xd = upload_bits(x)
        check_parity(_gemm(xd, w, m), x, w, label="gemm random codes")
        check_parity(_gemm(xd, w, m, torch.float32), x, w, label="gemm random codes fp32")


def test_dequant_bf16_bit_exact():
    # Expanded weights equal the oracle's, bit for bit: exact e4m3 x e2m1, and
    # t * e4m3 * e2m1 rounded once (ties to even) with the tensor scale.
    for n, k, t in [(64, 4096, 3.7e-5), (333, 1024, 0.25), (7, 16, 1.0)]:
        packed, scales = workload.random_codes(n, k, n * k)
        scales[0, :] = np.arange(scales.shape[1]) % 8          # subnormal scale bytes
        w = Weight(packed, scales, float(np.float32(t)))
        for apply_t in (False, True):
            got = _expanded(w, apply_t).cpu().numpy().view(np.uint16)
            want = oracle.dequant_bf16(packed, scales, w.t, apply_t)
            assert np.array_equal(got, want), (n, k, apply_t)


def test_expanded_gemm_equals_gemm():
    # Expand once (no tensor scale), then the bf16-weight product: the same
    # bits as the NVFP4 product, at a large M and on ragged shapes.
    for n, k, m in [(8192, 4096, 1536), (4136, 4096, 70), (333, 1024, 200)]:
        w = Weight.from_f32(workload.weights_f32(n, k, n + m))
        x = workload.activations_bf16(m, k, 91 + m)
        xd = upload_bits(x)
        ref = bits(_gemm(xd, w, m)).clone()
        wbf = _expanded(w, False)
        y = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
        st = nv.gemm_expanded_raw(xd.data_ptr(), wbf.data_ptr(), w.t, y.data_ptr(), m, n, k, nv.OUT_BF16, _stream())
        torch.cuda.synchronize()
        assert st == nv.OK
        assert torch.equal(bits(y), ref), (n, k, m)


def _library(xd, wbf, w, m, od=nv.OUT_BF16):
    y = torch.empty((m, w.n), dtype=torch.float32 if od == nv.OUT_F32 else torch.bfloat16, device=DEV)
    st = nv.gemm_library_raw(xd.data_ptr(), wbf.data_ptr(), w.t, y.data_ptr(), m, w.n, w.k, od, _stream())
    torch.cuda.synchronize()
    assert st == nv.OK, st
    return y


def test_library_gemm_parity_and_repeatability():
    # Expand once, then the library GEMM: within the oracle's tolerance (bf16
    # and fp32 outputs) on sampled columns of large and ragged shapes, and the
    # same bits on a second call of the same shape.
    for n, k, m in [(8192, 4096, 1536), (4136, 4096, 70), (333, 1024, 200), (24576, 4096, 33)]:
        w = Weight.from_f32(workload.weights_f32(n, k, n + m + 1))
        x = workload.activations_bf16(m, k, 93 + m)
        xd = upload_bits(x)
        wbf = _expanded(w, False)
        cols = np.unique(np.concatenate([np.arange(8), np.arange(n - 8, n), workload.rng(n).integers(0, n, 64)]))
        for od in (nv.OUT_BF16, nv.OUT_F32):
            y = _library(xd, wbf, w, m, od)
            check_parity(y, x, w, cols=cols, label=f"library gemm {n}x{k}")
            assert torch.equal(bits(_library(xd, wbf, w, m, od)), bits(y)), (n, k, m, od)


def test_library_gemm_in_a_graph_matches_eager():
    # After a first call outside capture, a captured call replays with the
    # eager call's bits, replay after replay, with eager work in between.
    n, k, m = 4096, 8192, 1100
    w = Weight.from_f32(workload.weights_f32(n, k, 17))
    xd = upload_bits(workload.activations_bf16(m, k, 18))
    wbf = _expanded(w, False)
    ref = bits(_library(xd, wbf, w, m)).clone()
    y = torch.full((m, n), -1.0, dtype=torch.bfloat16, device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            assert nv.gemm_library_raw(xd.data_ptr(), wbf.data_ptr(), w.t, y.data_ptr(), m, n, k, nv.OUT_BF16,
                                       s.cuda_stream) == nv.OK
    torch.cuda.synchronize()
    for _ in range(3):
        y.fill_(-1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(bits(y), ref)
        _library(xd, wbf, w, 64)


def test_library_gemm_contract_and_errors():
    w = Weight.from_f32(workload.weights_f32(64, 256, 3))
    wbf = _expanded(w, False)
    x = torch.zeros((3, 256), dtype=torch.bfloat16, device=DEV)
    y = torch.empty((3, 64), dtype=torch.bfloat16, device=DEV)
    s = _stream()
    assert nv.gemm_library_raw(x.data_ptr(), wbf.data_ptr(), w.t, y.data_ptr(), 0, 64, 256, nv.OUT_BF16, s) == nv.OK
    assert nv.gemm_library_raw(x.data_ptr(), wbf.data_ptr(), w.t, y.data_ptr(), 3, 64, 100, nv.OUT_BF16,
                               s) == nv.ERR_SHAPE
    assert nv.gemm_library_raw(x.data_ptr() + 2, wbf.data_ptr(), w.t, y.data_ptr(), 3, 64, 256, nv.OUT_BF16,
                               s) == nv.ERR_ALIGN
    assert nv.gemm_library_raw(x.data_ptr(), wbf.data_ptr(), w.t, y.data_ptr(), 3, 64, 256, 7, s) == nv.ERR_DTYPE
    assert nv.gemm_library_raw(x.data_ptr(), 0, w.t, y.data_ptr(), 3, 64, 256, nv.OUT_BF16, s) == nv.ERR_NULL


def test_matmul_expand_three_regimes():
    # Below the threshold nvfp4_matmul's bits (the scratch may be NULL); from
    # it on, the expanded weight through the library: the bits of
    # nvfp4_dequant_bf16 + nvfp4_gemm_library, within the oracle's tolerance.
    n, k = 4096, 4096
    w = Weight.from_f32(workload.weights_f32(n, k, 51))
    x = workload.activations_bf16(1100, k, 52)
    xd = upload_bits(x)
    scratch = torch.empty((n, k), dtype=torch.bfloat16, device=DEV)
    s = _stream()

    def run(m, scratch_ptr, threshold):
        y = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
        st = nv.matmul_expand_raw(xd.data_ptr(), w.wp.data_ptr(), w.sc.data_ptr(), w.t, y.data_ptr(), m, n, k,
                                  nv.OUT_BF16, scratch_ptr, threshold, s)
        torch.cuda.synchronize()
        assert st == nv.OK, st
        return y

    for m in (5, 64, 300):
        assert torch.equal(bits(run(m, 0, 0)), bits(_gemm(xd, w, m, fn=nv.matmul_raw))), m
    wbf = _expanded(w, False)
    for m, threshold in ((1100, 0), (300, 256)):
        y = run(m, scratch.data_ptr(), threshold)
        assert torch.equal(bits(y), bits(_library(xd, wbf, w, m))), (m, threshold)
        assert torch.equal(scratch.view(torch.int16), wbf), "scratch holds the expanded weight"
        cols = np.unique(np.concatenate([np.arange(8), workload.rng(53).integers(0, n, 64)]))
        check_parity(y, x[:m], w, cols=cols, label=f"matmul_expand M={m}")
    y = torch.empty((1100, n), dtype=torch.bfloat16, device=DEV)
    assert nv.matmul_expand_raw(xd.data_ptr(), w.wp.data_ptr(), w.sc.data_ptr(), w.t, y.data_ptr(), 1100, n, k,
                                nv.OUT_BF16, 0, 0, s) == nv.ERR_NULL
    assert nv.matmul_expand_raw(xd.data_ptr(), w.wp.data_ptr(), w.sc.data_ptr(), w.t, y.data_ptr(), 1100, n, k,
                                nv.OUT_BF16, scratch.data_ptr(), -1, s) == nv.ERR_SHAPE


def test_gemm_contract_and_errors():
    assert nv.gemm_shape_ok(0, 1, 256) and nv.gemm_shape_ok(4096, 8192, 4096)
    assert not nv.gemm_shape_ok(1, 1, 100) and not nv.gemm_shape_ok(-1, 1, 256)
    w = Weight.from_f32(workload.weights_f32(64, 256, 3))
    y = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    x = torch.empty((0, 256), dtype=torch.bfloat16, device=DEV)
    assert nv.gemm_raw(x.data_ptr(), w.wp.data_ptr(), w.sc.data_ptr(), w.t, y.data_ptr(), 0, 64, 256,
                       nv.OUT_BF16, _stream()) == nv.OK
    xr = torch.zeros((3, 256), dtype=torch.bfloat16, device=DEV)
    y3 = torch.empty((3, 64), dtype=torch.bfloat16, device=DEV)
    assert nv.gemm_raw(xr.data_ptr() + 2, w.wp.data_ptr(), w.sc.data_ptr(), w.t, y3.data_ptr(), 3, 64, 256,
                       nv.OUT_BF16, _stream()) == nv.ERR_ALIGN
    assert nv.gemm_raw(xr.data_ptr(), w.wp.data_ptr(), w.sc.data_ptr(), w.t, y3.data_ptr(), 3, 64, 256,
                       7, _stream()) == nv.ERR_DTYPE
    assert nv.gemm_raw(xr.data_ptr(), 0, w.sc.data_ptr(), w.t, y3.data_ptr(), 3, 64, 256,
                       nv.OUT_BF16, _stream()) == nv.ERR_NULL
