"""Parity of the other regimes and forms at the sizes the benchmark times them
(gpu): two 12288x4096 projections over one x, the silu input on 4096x12288,
the de-interleaved Q|K|V|Z store on 12288x4096, a grouped launch over 128
experts of 1536x4096, the FP8 product on every decode-round shape at 1, 16
and 32 rows and its GEMM at 64 and 1024 rows, and the expanded weight of
8192x4096.  The oracle computes
sampled columns (or rows) one by one; the launches are the ones the benchmark
makes."""
import numpy as np
import pytest
import torch

import oracle
import verify_nvfp4_w4a16_amd as nv
import workload
from tests._gpu import DEV, Weight, bits, check_parity, to_f64, upload_bits, upload_u8

pytestmark = pytest.mark.gpu


def _s():
    return torch.cuda.current_stream().cuda_stream


def _cols(n, seed, count=48):
    return np.unique(np.concatenate([np.arange(4), np.arange(n - 4, n), workload.rng(seed).integers(0, n, count)]))


def test_dual_at_bench_size():
    n, k, m = 12288, 4096, 8
    w0 = Weight.from_f32(workload.weights_f32(n, k, 11))
    w1 = Weight.from_f32(workload.weights_f32(n, k, 12))
    x = workload.activations_bf16(m, k, 13)
    xd = upload_bits(x)
    y0 = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
    y1 = torch.empty_like(y0)
    assert nv.linear_dual_raw(xd.data_ptr(), w0.wp.data_ptr(), w0.sc.data_ptr(), w0.t, y0.data_ptr(),
                              w1.wp.data_ptr(), w1.sc.data_ptr(), w1.t, y1.data_ptr(), m, n, k, nv.OUT_BF16,
                              _s()) == nv.OK
    torch.cuda.synchronize()
    cols = _cols(n, 1)
    check_parity(y0, x, w0, cols=cols, label="dual 12288x4096 M=8 weight 0")
    check_parity(y1, x, w1, cols=cols, label="dual 12288x4096 M=8 weight 1")


def test_silu_input_at_bench_size():
    n, k = 4096, 12288
    w = Weight.from_f32(workload.weights_f32(n, k, 14))
    for m in (1, 2):
        g, u = workload.activations_bf16(m, k, 15), workload.activations_bf16(m, k, 16)
        y = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
        assert nv.linear_silu_input_raw(upload_bits(g).data_ptr(), upload_bits(u).data_ptr(), w.wp.data_ptr(),
                                        w.sc.data_ptr(), w.t, y.data_ptr(), m, n, k, nv.OUT_BF16, _s()) == nv.OK
        torch.cuda.synchronize()
        check_parity(y, oracle.silu_mul_bf16(g, u), w, cols=_cols(n, 2), label=f"silu input 4096x12288 M={m}")


def test_qkvz_store_at_bench_size():
    n, k, m, widths = 12288, 4096, 8, [256, 128, 128, 256]
    w = Weight.from_f32(workload.weights_f32(n, k, 17))
    x = workload.activations_bf16(m, k, 18)
    y = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
    assert nv.linear_deinterleave_raw(upload_bits(x).data_ptr(), w.wp.data_ptr(), w.sc.data_ptr(), w.t,
                                      y.data_ptr(), m, n, k, nv.OUT_BF16, widths, _s()) == nv.OK
    torch.cuda.synchronize()
    rows = _cols(n, 3)                                   # weight rows, sampled
    out = oracle.deinterleave_columns(n, widths)          # output column of each weight row
    got = y[:, torch.from_numpy(out[rows]).to(DEV)]
    y_ref = oracle.linear_ref(x, w.packed, w.scales, w.t, rows)
    bnd = oracle.bound(x, w.packed, w.scales, w.t, rows)
    viol = oracle.max_violation(to_f64(got), y_ref, bnd, "bf16")
    assert viol <= 1.0, viol


def test_grouped_128_experts_at_bench_size():
    experts, n, k, m = 128, 1536, 4096, 2
    w = Weight.from_f32(workload.weights_f32(n, k, 19))
    xs = [workload.activations_bf16(m, k, 20 + e % 4) for e in range(experts)]
    xd = [upload_bits(x) for x in xs]
    ys = [torch.empty((m, n), dtype=torch.bfloat16, device=DEV) for _ in range(experts)]
    rec = np.zeros(experts, dtype=nv.GROUP_DTYPE)
    for e in range(experts):
        rec[e] = (xd[e].data_ptr(), w.wp.data_ptr(), w.sc.data_ptr(), ys[e].data_ptr(), w.t, m)
    table = upload_u8(rec.view(np.uint8))
    assert nv.linear_grouped_raw(table.data_ptr(), experts, m, n, k, nv.OUT_BF16, _s()) == nv.OK
    torch.cuda.synchronize()
    cols = _cols(n, 4)
    for e in (0, 1, 2, 3, 127):
        check_parity(ys[e], xs[e], w, cols=cols, label=f"grouped expert {e}")
    for e in range(4, experts):                            # same x and weight as expert e % 4
        assert torch.equal(bits(ys[e]), bits(ys[e % 4])), e


@pytest.mark.parametrize("shape", workload.ROUND_SHAPES, ids=lambda s: f"{s.n}x{s.k}")
def test_fp8_at_bench_size(shape):
    codes, scales = nv.fp8_pack(workload.weights_f32(shape.n, shape.k, 21))
    wd, sd = upload_u8(codes), torch.from_numpy(scales).to(DEV)
    cols = _cols(shape.n, 5)
    # the oracle on the 128-row scale blocks that hold the sampled columns
    blocks = np.unique(cols // 128)
    sub_codes = np.concatenate([codes[128 * b:128 * (b + 1)] for b in blocks])
    sub_scales = scales[blocks]
    sub_cols = np.searchsorted(blocks, cols // 128) * 128 + cols % 128
    for m in (1, 16, 32):
        x = workload.activations_bf16(m, shape.k, 22)
        y = torch.empty((m, shape.n), dtype=torch.bfloat16, device=DEV)
        assert nv.fp8_linear_raw(upload_bits(x).data_ptr(), wd.data_ptr(), sd.data_ptr(), y.data_ptr(), m,
                                 shape.n, shape.k, nv.OUT_BF16, _s()) == nv.OK
        torch.cuda.synchronize()
        ref = oracle.linear_fp8_ref(x, sub_codes, sub_scales, sub_cols)
        bnd = oracle.bound_fp8(x, sub_codes, sub_scales, sub_cols)
        viol = oracle.max_violation(to_f64(y)[:, cols], ref, bnd, "bf16")
        print(f"[parity] fp8 {shape.n}x{shape.k} M={m} max err/tol = {viol:.3g}", flush=True)
        assert viol <= 1.0, (m, viol)
        # the many-row GEMM gives every row the same bits
        yg = torch.empty_like(y)
        assert nv.fp8_gemm_raw(upload_bits(x).data_ptr(), wd.data_ptr(), sd.data_ptr(), yg.data_ptr(), m,
                               shape.n, shape.k, nv.OUT_BF16, _s()) == nv.OK
        torch.cuda.synchronize()
        assert torch.equal(bits(yg), bits(y)), m


def test_expanded_weight_at_bench_size():
    n, k = 8192, 4096
    packed, scales, t = nv.pack(workload.weights_f32(n, k, 9))
    dst = torch.empty((n, k), dtype=torch.int16, device=DEV)
    for apply_t in (0, 1):
        assert nv.dequant_bf16_raw(upload_u8(packed).data_ptr(), upload_u8(scales).data_ptr(), t, apply_t,
                                   dst.data_ptr(), n, k, _s()) == nv.OK
        torch.cuda.synchronize()
        rows = _cols(n, 6, 64)
        got = dst[torch.from_numpy(rows).to(DEV)].cpu().numpy().view(np.uint16)
        want = oracle.dequant_bf16(packed[rows], scales[rows], t, bool(apply_t))
        assert np.array_equal(got, want), apply_t


@pytest.mark.parametrize("shape", workload.ROUND_SHAPES, ids=lambda s: f"{s.n}x{s.k}")
def test_fp8_gemm_at_bench_size(shape):
    codes, scales = nv.fp8_pack(workload.weights_f32(shape.n, shape.k, 21))
    wd, sd = upload_u8(codes), torch.from_numpy(scales).to(DEV)
    cols = _cols(shape.n, 7)
    blocks = np.unique(cols // 128)
    sub_codes = np.concatenate([codes[128 * b:128 * (b + 1)] for b in blocks])
    sub_scales = scales[blocks]
    sub_cols = np.searchsorted(blocks, cols // 128) * 128 + cols % 128
    for m in (64, 1024):
        x = workload.activations_bf16(m, shape.k, 23)
        y = torch.empty((m, shape.n), dtype=torch.bfloat16, device=DEV)
        assert nv.fp8_gemm_raw(upload_bits(x).data_ptr(), wd.data_ptr(), sd.data_ptr(), y.data_ptr(), m,
                               shape.n, shape.k, nv.OUT_BF16, _s()) == nv.OK
        torch.cuda.synchronize()
        ref = oracle.linear_fp8_ref(x, sub_codes, sub_scales, sub_cols)
        bnd = oracle.bound_fp8(x, sub_codes, sub_scales, sub_cols)
        viol = oracle.max_violation(to_f64(y)[:, cols], ref, bnd, "bf16")
        print(f"[parity] fp8 gemm {shape.n}x{shape.k} M={m} max err/tol = {viol:.3g}", flush=True)
        assert viol <= 1.0, (m, viol)
