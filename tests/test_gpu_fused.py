"""Fused and grouped forms of the product on the GPU (gpu): two projections
over one x, the silu(gate) * up input, de-interleaved Q|gate and Q|K|V|Z
outputs, and a grouped launch over a device table.  Each output is
bit-identical to nvfp4_linear's for the same row, x and weight, and within
the oracle's tolerance."""
import numpy as np
import pytest
import torch

import oracle
import verify_nvfp4_w4a16_amd as nv
import workload
from tests._gpu import DEV, Weight, bits, check_parity, upload_bits, upload_u8

pytestmark = pytest.mark.gpu


def _s():
    return torch.cuda.current_stream().cuda_stream


def _linear(xd, w, m, out_dtype=torch.bfloat16):
    y = torch.empty((m, w.n), dtype=out_dtype, device=DEV)
    od = nv.OUT_F32 if out_dtype == torch.float32 else nv.OUT_BF16
    assert nv.linear_raw(xd.data_ptr(), w.wp.data_ptr(), w.sc.data_ptr(), w.t, y.data_ptr(), m, w.n, w.k, od,
                         _s()) == nv.OK
    torch.cuda.synchronize()
    return y


def test_dual_equals_two_products():
    for n, k in [(4096, 4096), (4136, 2048)]:
        w0 = Weight.from_f32(workload.weights_f32(n, k, 11))
        w1 = Weight.from_f32(workload.weights_f32(n, k, 12))
        for m in (1, 2, 3, 17, 32):
            x = workload.activations_bf16(m, k, 13 + m)
            xd = upload_bits(x)
            y0 = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
            y1 = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
            st = nv.linear_dual_raw(xd.data_ptr(), w0.wp.data_ptr(), w0.sc.data_ptr(), w0.t, y0.data_ptr(),
                                    w1.wp.data_ptr(), w1.sc.data_ptr(), w1.t, y1.data_ptr(), m, n, k, nv.OUT_BF16,
                                    _s())
            torch.cuda.synchronize()
            assert st == nv.OK
            assert torch.equal(bits(y0), bits(_linear(xd, w0, m))), (n, m)
            assert torch.equal(bits(y1), bits(_linear(xd, w1, m))), (n, m)
            if m in (3, 32):
                check_parity(y1, x, w1, label=f"dual {n}x{k}")


def _identity_weight(k):
    # W[n, n] = 1 (e2m1 code 2 at scale 1.0), zero elsewhere: y = x exactly
    packed = np.zeros((k, k // 2), np.uint8)
    idx = np.arange(k)
    packed[idx, idx // 2] = np.where(idx % 2 == 0, 0x02, 0x20).astype(np.uint8)
    return Weight(packed, np.full((k, k // 16), 0x38, np.uint8), 1.0)


def _silu(gd, ud, w, m, out_dtype=torch.bfloat16):
    y = torch.empty((m, w.n), dtype=out_dtype, device=DEV)
    od = nv.OUT_F32 if out_dtype == torch.float32 else nv.OUT_BF16
    st = nv.linear_silu_input_raw(gd.data_ptr(), ud.data_ptr(), w.wp.data_ptr(), w.sc.data_ptr(), w.t,
                                  y.data_ptr(), m, w.n, w.k, od, _s())
    torch.cuda.synchronize()
    assert st == nv.OK, st
    return y


def test_silu_input_forms_the_activation_once_and_multiplies_it():
    k, n = 4096, 4096
    m = 32                                           # every row count of the contract
    g = workload.activations_bf16(m, k, 21)
    u = workload.activations_bf16(m, k, 22, outliers=True)
    gd, ud = upload_bits(g), upload_bits(u)
    # the activation the kernel forms, read back through an identity weight
    h_gpu = _silu(gd, ud, _identity_weight(k), m, torch.float32).cpu().numpy()
    h_bits = workload.f32_to_bf16_bits(h_gpu)
    assert np.array_equal(workload.bf16_bits_to_f32(h_bits), h_gpu)          # it is a bf16 vector
    h_ref = oracle.silu_mul_bf16(g, u)
    off = h_bits != h_ref
    # fp32 silu(g) * u rounded to bf16 against the float64 one: a bf16 step
    # apart at most, and only where the value sits next to a rounding midpoint
    assert off.mean() < 2e-3, off.mean()
    assert np.all(np.abs(h_bits.astype(np.int32)[off] - h_ref.astype(np.int32)[off]) == 1)
    # at one row the activation is formed inside the product's kernel: the
    # same bits as the activation formed first (here read back through the
    # identity weight), also for gate values where silu saturates or vanishes
    edge = g[:1].copy()
    edge[0, :8] = workload.f32_to_bf16_bits(np.array([0.0, -0.0, 1e-30, -1e-30, 88.0, -88.0, 1e4, -1e4],
                                                    dtype=np.float32))
    ed = upload_bits(edge)
    h_one = _silu(ed, ud[:1], _identity_weight(k), 1, torch.float32)
    h_two = _silu(torch.cat([ed, ed]), torch.cat([ud[:1], ud[:1]]), _identity_weight(k), 2, torch.float32)
    assert torch.equal(bits(h_one), bits(h_two[:1]))
    # the fused product equals nvfp4_linear on that activation, bit for bit
    w = Weight.from_f32(workload.weights_f32(n, k, 23))
    for mm in (1, 3, 7, 8, 17, 32):
        y = _silu(gd, ud, w, mm)
        assert torch.equal(bits(y), bits(_linear(upload_bits(h_bits[:mm]), w, mm))), mm
    check_parity(_silu(gd, ud, w, m), h_ref, w, label="silu input M=32")
    check_parity(_silu(gd, ud, w, 5, torch.float32), h_ref[:5], w, label="silu input M=5 fp32")
    # more rows than the contract allows is refused
    st = nv.linear_silu_input_raw(gd.data_ptr(), ud.data_ptr(), w.wp.data_ptr(), w.sc.data_ptr(), w.t,
                                  gd.data_ptr(), 33, n, k, nv.OUT_BF16, _s())
    assert st == nv.ERR_SHAPE


@pytest.mark.parametrize("n,widths", [(8192, [128, 128]), (12288, [256, 128, 128, 256]), (4104, [3, 5, 1, 10])],
                         ids=["qg", "qkvz", "odd"])
def test_deinterleaved_output_is_a_column_permutation(n, widths):
    k = 4096
    w = Weight.from_f32(workload.weights_f32(n, k, 31 + n))
    cols = torch.from_numpy(oracle.deinterleave_columns(n, widths)).to(DEV)
    for m in (1, 4, 32):
        x = workload.activations_bf16(m, k, 32 + m)
        xd = upload_bits(x)
        y = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
        st = nv.linear_deinterleave_raw(xd.data_ptr(), w.wp.data_ptr(), w.sc.data_ptr(), w.t, y.data_ptr(), m, n,
                                        k, nv.OUT_BF16, widths, _s())
        torch.cuda.synchronize()
        assert st == nv.OK
        plain = bits(_linear(xd, w, m))
        want = torch.empty_like(plain)
        want[:, cols] = plain
        assert torch.equal(bits(y), want), (n, m)
    bad = nv.linear_deinterleave_raw(xd.data_ptr(), w.wp.data_ptr(), w.sc.data_ptr(), w.t, y.data_ptr(), 1, n,
                                     k, nv.OUT_BF16, [n + 1], _s())
    assert bad == nv.ERR_SHAPE


def test_grouped_launch_over_a_device_table():
    # Eight experts of 1536 x 4096 with 0..32 routed rows each, one launch:
    # every expert's output equals nvfp4_linear's, bit for bit; a zero-row
    # expert's output is left untouched.
    n, k = 1536, 4096
    rows = [0, 1, 2, 3, 5, 8, 13, 32]
    ws = [Weight.from_f32(workload.weights_f32(n, k, 40 + e)) for e in range(len(rows))]
    xs = [upload_bits(workload.activations_bf16(max(m, 1), k, 50 + e)) for e, m in enumerate(rows)]
    ys = [torch.full((max(m, 1), n), -7.0, dtype=torch.float32, device=DEV) for m in rows]
    rec = np.zeros(len(rows), dtype=nv.GROUP_DTYPE)
    for e, m in enumerate(rows):
        rec[e] = (xs[e].data_ptr(), ws[e].wp.data_ptr(), ws[e].sc.data_ptr(), ys[e].data_ptr(), ws[e].t, m)
    table = upload_u8(rec.view(np.uint8))
    st = nv.linear_grouped_raw(table.data_ptr(), len(rows), max(rows), n, k, nv.OUT_F32, _s())
    torch.cuda.synchronize()
    assert st == nv.OK
    for e, m in enumerate(rows):
        if m == 0:
            assert bool((ys[e] == -7.0).all())
            continue
        assert torch.equal(bits(ys[e]), bits(_linear(xs[e], ws[e], m, torch.float32))), e
    check_parity(ys[-1], workload.activations_bf16(32, k, 50 + len(rows) - 1), ws[-1], label="grouped expert M=32")


def test_grouped_launch_beyond_the_exchange_workspace():
    # Forty experts at up to 17 rows: the many-row kernel's exchange regions
    # for every expert would not fit the device workspace, so the launch runs
    # another kernel of the same tile; each expert's rows still have the bits
    # nvfp4_linear gives them alone (where the exchange fits).
    n, k, count = 1536, 4096, 40
    w = Weight.from_f32(workload.weights_f32(n, k, 60))
    rows = [17 - (e % 17) for e in range(count)]
    xs = [upload_bits(workload.activations_bf16(m, k, 61 + e)) for e, m in enumerate(rows)]
    ys = [torch.empty((m, n), dtype=torch.bfloat16, device=DEV) for m in rows]
    rec = np.zeros(count, dtype=nv.GROUP_DTYPE)
    for e, m in enumerate(rows):
        rec[e] = (xs[e].data_ptr(), w.wp.data_ptr(), w.sc.data_ptr(), ys[e].data_ptr(), w.t, m)
    table = upload_u8(rec.view(np.uint8))
    st = nv.linear_grouped_raw(table.data_ptr(), count, max(rows), n, k, nv.OUT_BF16, _s())
    torch.cuda.synchronize()
    assert st == nv.OK
    for e in (0, 1, 16, 17, 39):
        assert torch.equal(bits(ys[e]), bits(_linear(xs[e], w, rows[e]))), e
