"""Parity of the HIP path with the fp64 oracle on the workloads' shapes, and
bit-exact row invariance across M = 1..32 (gpu)."""
import numpy as np
import pytest
import torch

import oracle
import verify_nvfp4_w4a16_amd as nv
import workload
from tests._gpu import DEV, Weight, bits, check_parity, run, to_f64, upload_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def inv_weight():
    s = workload.INVARIANCE
    return Weight.from_f32(workload.weights_f32(s.n, s.k, workload.SEEDS["invariance"][0]))


@pytest.fixture(scope="module")
def inv_x():
    return workload.activations_bf16(32, workload.INVARIANCE.k, workload.SEEDS["invariance"][1])


def test_single_linear_parity():
    s = workload.SINGLE
    ws, xs = workload.SEEDS["single"]
    w = Weight.from_f32(workload.weights_f32(s.n, s.k, ws))
    x = workload.activations_bf16(1, s.k, xs)
    check_parity(run(x, w), x, w, label="single 1024x1024")


def test_invariance_parity_every_m(inv_weight, inv_x):
    w = inv_weight
    y_ref = oracle.linear_ref(inv_x, w.packed, w.scales, w.t)
    bnd = oracle.bound(inv_x, w.packed, w.scales, w.t)
    worst = 0.0
    for m in range(1, 33):
        y = run(inv_x[:m], w)
        viol = oracle.max_violation(to_f64(y), y_ref[:m], bnd[:m], "bf16")
        worst = max(worst, viol)
        assert viol <= 1.0, f"M={m}: max err/tol {viol}"
    print(f"[parity] invariance 4096x4096 M=1..32 worst err/tol = {worst:.3g}", flush=True)


def test_row_invariance_bit_exact(inv_weight, inv_x):
    w = inv_weight
    alone = [bits(run(inv_x[r:r + 1], w))[0].clone() for r in range(32)]
    for m in range(1, 33):
        y = bits(run(inv_x[:m], w))
        for r in range(m):
            assert torch.equal(y[r], alone[r]), f"row {r} differs at M={m}"
    # a row's bits do not depend on its position either
    x_rev = np.ascontiguousarray(inv_x[::-1])
    y = bits(run(x_rev, w))
    for r in range(32):
        assert torch.equal(y[31 - r], alone[r])
    print("[invariance] 4096x4096: every row bit-identical at M=1..32 and any position", flush=True)


def test_qkv_outliers_parity_and_invariance():
    s = workload.QKV
    ws, xs = workload.SEEDS["qkv"]
    w = Weight.from_f32(workload.weights_f32(s.n, s.k, ws))
    x = workload.activations_bf16(32, s.k, xs, outliers=True)
    check_parity(run(x, w), x, w, label="qkv 12288x4096 outliers")
    check_parity(run(x[:16], w), x[:16], w, label="qkv 12288x4096 outliers")
    alone = [bits(run(x[r:r + 1], w))[0].clone() for r in range(32)]
    for m in range(16, 33):
        y = bits(run(x[:m], w))
        for r in range(m):
            assert torch.equal(y[r], alone[r]), f"row {r} differs at M={m}"


def test_round_shapes_parity():
    # The decode round's shapes at its row counts, and at every row count the
    # kernel choice distinguishes (per-tile kernel with one or more chunk
    # buffers, persistent, many-row with one or two windows requested at
    # once): each row of a 32-row block, computed at M rows, is bit-equal to
    # the same row computed alone, and within the oracle's tolerance.
    rng = workload.rng(77)
    for proj, s in enumerate(workload.ROUND_SHAPES):
        w = Weight.from_f32(workload.weights_f32(s.n, s.k, workload.round_weight_seed(0, proj)))
        cols = np.unique(np.concatenate([np.arange(64), np.arange(s.n - 64, s.n),
                                         rng.integers(0, s.n, 1024)]))
        for m in workload.ROUND_M:
            x = workload.activations_bf16(m, s.k, workload.round_act_seed(0, proj, m))
            check_parity(run(x, w), x, w, cols=cols, label=f"round proj{proj}")
        xb = workload.activations_bf16(32, s.k, workload.round_act_seed(0, proj, 99))
        alone = torch.cat([bits(run(xb[r:r + 1], w)) for r in range(32)])
        for m in (2, 3, 4, 5, 6, 7, 8, 12, 16, 17, 24, 32):
            y = run(xb[:m], w)
            assert torch.equal(bits(y), alone[:m]), f"round proj{proj} M={m}: rows differ from M=1"
            if m <= 8:
                check_parity(y, xb[:m], w, cols=cols, label=f"round proj{proj} block")


def test_head_fp32_parity_and_gemv_vs_mfma_rows():
    # The output head (151552 x 4096, fp32 logits) at every row count from 1
    # to 32: each M's rows are bit-identical to the 32-row product's first M
    # rows (so row 0 equals the one-row product), and the values are within
    # the oracle's tolerance on sampled columns at the row counts where the
    # kernel choice changes (per-tile kernel at 1, many-row kernel at 2..4
    # because each CU would run many per-tile rounds, ...).
    s = workload.HEAD
    ws, xs = workload.SEEDS["head"]
    w = Weight.from_f32(workload.weights_f32(s.n, s.k, ws))
    x = workload.activations_bf16(32, s.k, xs)
    rng = workload.rng(78)
    cols = np.unique(np.concatenate([np.arange(64), np.arange(s.n - 64, s.n),
                                     rng.integers(0, s.n, 2048)]))
    y32 = run(x, w, torch.float32)
    check_parity(y32, x, w, cols=cols, label="head fp32 M=32")
    ref = bits(y32).clone()
    for m in range(1, 32):
        y = run(x[:m], w, torch.float32)
        assert torch.equal(bits(y), ref[:m]), f"head: rows at M={m} differ from the 32-row product"
        if m in (1, 2, 3, 4, 5, 8, 16, 17):
            check_parity(y, x[:m], w, cols=cols, label=f"head fp32 M={m}")
    print("[invariance] head: rows at every M = 1..31 bit-identical to the M=32 product "
          "(M=1 GEMV row == M=32 row 0)", flush=True)


def test_random_codes_full_scale_range():
    # Every e2m1 code and every finite non-negative scale byte, incl. subnormal
    # scales and zero groups, with a ragged N.
    for n, k, m in [(1, 256, 1), (17, 256, 3), (333, 1024, 32), (1000, 2048, 16), (4111, 512, 19)]:
        packed, scales = workload.random_codes(n, k, n + k)
        scales[:, ::5] = 0
        w = Weight(packed, scales, 0.0371)
        x = workload.activations_bf16(m, k, n * 3 + m, outliers=True)
        check_parity(run(x, w), x, w, label="random codes")
        check_parity(run(x, w, torch.float32), x, w, label="random codes fp32")


def test_nan_scale_propagates_like_the_oracle():
    n, k = 40, 256
    packed, scales = workload.random_codes(n, k, 5)
    scales[7, 3] = 0x7F
    w = Weight(packed, scales, 1.0)
    x = workload.activations_bf16(2, k, 6)
    y = to_f64(run(x, w, torch.float32))
    assert np.isnan(y[:, 7]).all() and not np.isnan(np.delete(y, 7, axis=1)).any()
    check_parity(run(x, w, torch.float32), x, w, label="nan scale")


def test_bf16_output_is_rounded_fp32_output(inv_weight, inv_x):
    y32 = run(inv_x[:7], inv_weight, torch.float32)
    y16 = run(inv_x[:7], inv_weight, torch.bfloat16)
    assert torch.equal(y32.to(torch.bfloat16).view(torch.int16), y16.view(torch.int16))


def test_launch_settings_never_change_bits():
    # Only the K segmentation (waves) and its grouping (split) enter the
    # arithmetic: every cols/unroll/mwaves choice and every kernel that can
    # run the shape gives the default tile's bits.
    s = workload.INVARIANCE
    w = Weight.from_f32(workload.weights_f32(s.n, s.k, 61))
    base = nv.table_tile(s.n, s.k)
    for m in (1, 3, 17, 32):
        x = upload_bits(workload.activations_bf16(m, s.k, 62 + m))
        ref = bits(nv.linear(x, w.wp, w.sc, w.t)).clone()
        ran = set()
        for kernel in (nv.KERNEL_PERSISTENT, nv.KERNEL_TILE, nv.KERNEL_SPLIT, nv.KERNEL_GENERIC, nv.KERNEL_WHOLE):
            for cols in (16, 32, 64):
                for unroll in (1, 2, 4):
                    for mwaves in (4, 6, 8):
                        if s.k % (128 * unroll * base.waves):
                            continue
                        tile = base.replace(cols=cols, unroll=unroll, mwaves=mwaves, kernel=kernel)
                        y = torch.empty((m, s.n), dtype=torch.bfloat16, device=x.device)
                        st = nv.linear_tiled_raw(x.data_ptr(), w.wp.data_ptr(), w.sc.data_ptr(), w.t,
                                                 y.data_ptr(), m, s.n, s.k, nv.OUT_BF16, tile,
                                                 torch.cuda.current_stream().cuda_stream)
                        if st == nv.ERR_TILE:
                            continue                  # this kernel cannot run this shape
                        assert st == nv.OK
                        torch.cuda.synchronize()
                        ran.add(kernel)
                        assert torch.equal(bits(y), ref), f"M={m} {tile}"
        assert nv.KERNEL_GENERIC in ran and nv.KERNEL_SPLIT in ran, (m, ran)
        if m <= 3:
            assert nv.KERNEL_TILE in ran and nv.KERNEL_PERSISTENT in ran, (m, ran)


def _run_tiled(xd, w, m, tile, out_dtype=torch.bfloat16):
    y = torch.empty((m, w.n), dtype=out_dtype, device=DEV)
    st = nv.linear_tiled_raw(xd.data_ptr(), w.wp.data_ptr(), w.sc.data_ptr(), w.t, y.data_ptr(), m, w.n, w.k,
                             nv.OUT_F32 if out_dtype == torch.float32 else nv.OUT_BF16, tile,
                             torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return st, y


def test_ragged_columns_every_kernel_and_split():
    # N = 4136: the last column group of every kernel is partly past N (its
    # loads repeat row N-1, its stores are skipped).  For each segment
    # grouping (split 1, 2, 4, 8; above 1 the many-row kernel's groups meet
    # across workgroups; split 4 gives two-window groups, which one row tile
    # requests together) every kernel that can run the shape gives the same
    # bits, within the oracle's tolerance.
    n, k = 4136, 4096
    w = Weight.from_f32(workload.weights_f32(n, k, 91))
    for split in (1, 2, 4, 8):
        base = nv.table_tile(n, k).replace(split=split)
        for m in (1, 3, 16, 17, 32):
            x = workload.activations_bf16(m, k, 92 + m)
            xd = upload_bits(x)
            outs = {}
            for kernel in (nv.KERNEL_TILE, nv.KERNEL_PERSISTENT, nv.KERNEL_SPLIT, nv.KERNEL_GENERIC, nv.KERNEL_WHOLE):
                st, y = _run_tiled(xd, w, m, base.replace(kernel=kernel))
                if st == nv.ERR_TILE:
                    continue
                assert st == nv.OK
                outs[kernel] = y
            assert nv.KERNEL_SPLIT in outs and nv.KERNEL_GENERIC in outs
            first = next(iter(outs.values()))
            for kernel, y in outs.items():
                assert torch.equal(bits(y), bits(first)), f"split={split} M={m} kernel {kernel}"
            check_parity(first, x, w, label=f"ragged 4136x4096 split={split}")


def test_exhaustive_decode_every_code_and_scale_byte():
    # One-hot activations pick single weights, so y[m, n] = E2M1[m] * E4M3[n]
    # exactly (t = 1, fp32 output): all 16 e2m1 codes against all 256 scale
    # bytes (negative ones decoded literally, 0x7F/0xFF give NaN), through
    # every kernel that can run the shape.  Zeros compare as values (a -0
    # product lands in a +0 accumulator).
    from oracle.formats import E2M1, E4M3
    n, k = 256, 4096
    packed = np.zeros((n, k // 2), dtype=np.uint8)
    for j in range(8):
        packed[:, j] = (2 * j) | ((2 * j + 1) << 4)      # k = 0..15 hold codes 0..15
    scales = np.zeros((n, k // 16), dtype=np.uint8)
    scales[:, 0] = np.arange(256, dtype=np.uint8)
    w = Weight(packed, scales, 1.0)
    x = np.zeros((16, k), dtype=np.uint16)
    x[np.arange(16), np.arange(16)] = 0x3F80             # x[m, m] = 1.0
    expect = (E2M1[:, None] * E4M3[None, :]).astype(np.float32)
    xt = upload_bits(x)
    ran = 0
    for kernel in (nv.KERNEL_AUTO, nv.KERNEL_PERSISTENT, nv.KERNEL_TILE, nv.KERNEL_SPLIT, nv.KERNEL_GENERIC, nv.KERNEL_WHOLE):
        for m in (1, 16):
            y = torch.empty((m, n), dtype=torch.float32, device=DEV)
            st = nv.linear_tiled_raw(xt.data_ptr(), w.wp.data_ptr(), w.sc.data_ptr(), w.t, y.data_ptr(), m, n, k,
                                     nv.OUT_F32, nv.table_tile(n, k).replace(kernel=kernel),
                                     torch.cuda.current_stream().cuda_stream)
            if st == nv.ERR_TILE:
                continue
            assert st == nv.OK
            torch.cuda.synchronize()
            got = y.cpu().numpy()
            want = expect[:m]
            nan = np.isnan(want)
            assert np.array_equal(np.isnan(got), nan), (kernel, m)
            assert np.array_equal(got[~nan], want[~nan]), (kernel, m)
            ran += 1
    print(f"[decode] 16 codes x 256 scale bytes exact through {ran} kernel/row-count runs", flush=True)
    assert ran >= 6
