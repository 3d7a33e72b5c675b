"""The shape contract's limits through the HIP path (gpu): K = 2^20 with a
ragged N, N = 2^28 (weight offsets past 2^32 bytes), and one output column
with the smallest K."""
import numpy as np
import pytest
import torch

import oracle
import verify_nvfp4_w4a16_amd as nv
import workload
from tests._gpu import DEV, Weight, bits, check_parity, to_f64, upload_bits, upload_u8

pytestmark = pytest.mark.gpu

MAX_K = 1 << 20
MAX_N = 1 << 28


def _launch(xd, wp, sc, t, m, n, k, tile=None, out_dtype=torch.bfloat16):
    y = torch.empty((m, n), dtype=out_dtype, device=DEV)
    od = nv.OUT_F32 if out_dtype == torch.float32 else nv.OUT_BF16
    stream = torch.cuda.current_stream().cuda_stream
    if tile is None:
        st = nv.linear_raw(xd.data_ptr(), wp.data_ptr(), sc.data_ptr(), t, y.data_ptr(), m, n, k, od, stream)
    else:
        st = nv.linear_tiled_raw(xd.data_ptr(), wp.data_ptr(), sc.data_ptr(), t, y.data_ptr(), m, n, k, od, tile,
                                 stream)
    torch.cuda.synchronize()
    return st, y


def test_largest_k_every_kernel():
    # K = 2^20 (the contract's largest) with N = 40: one column group, its
    # last 24 columns past N; segments of 131072 k.  Every kernel that can
    # run the shape gives the same bits, each row's bits are those it gets
    # alone, and the result is within the oracle's tolerance.
    n, k = 40, MAX_K
    packed, scales = workload.random_codes(n, k, 71)
    w = Weight(packed, scales, 2.0 ** -9)
    x = workload.activations_bf16(32, k, 72)
    xd = upload_bits(x)
    alone = None
    for m in (1, 17, 32):
        outs = {}
        for kernel in (nv.KERNEL_AUTO, nv.KERNEL_TILE, nv.KERNEL_PERSISTENT, nv.KERNEL_SPLIT, nv.KERNEL_GENERIC, nv.KERNEL_WHOLE):
            st, y = _launch(xd, w.wp, w.sc, w.t, m, n, k, nv.table_tile(n, k).replace(kernel=kernel))
            if st == nv.ERR_TILE:
                continue                                  # x does not fit this kernel's LDS
            assert st == nv.OK, (m, kernel, st)
            outs[kernel] = y
        assert {nv.KERNEL_AUTO, nv.KERNEL_SPLIT, nv.KERNEL_GENERIC} <= set(outs), (m, sorted(outs))
        ref = bits(outs[nv.KERNEL_AUTO])
        for kernel, y in outs.items():
            assert torch.equal(bits(y), ref), f"M={m} kernel {kernel}"
        if alone is None:
            alone = ref[:1].clone()
        assert torch.equal(ref[:1], alone), f"row 0 at M={m} differs from M=1"
        check_parity(outs[nv.KERNEL_AUTO], x[:m], w, label=f"K=2^20 M={m}")


def test_largest_n_sampled_columns():
    # N = 2^28 with K = 256 (36 GiB of packed weights and scales): row n
    # holds row n % 4099 of a random block, so a weight or scale offset that
    # wrapped at 2^32 bytes (row 2^25 onwards) would read another row of the
    # block and fail on the sampled columns past it.  Columns are checked
    # against the oracle of the block rows; row 0 must equal its M = 1 bits.
    n, k, period = MAX_N, 256, 4099
    packed, scales = workload.random_codes(period, k, 81)
    t = 2.0 ** -7
    reps = -(-n // period)
    wp = upload_u8(packed).repeat(reps, 1)[:n]            # contiguous prefix rows
    sc = upload_u8(scales).repeat(reps, 1)[:n]
    assert wp.is_contiguous() and sc.is_contiguous()
    g = np.random.default_rng(82)
    cols = np.unique(np.concatenate([
        [0, 1, period - 1, period, (1 << 25) - 1, 1 << 25, (1 << 25) + 1, (1 << 26) + 5, (1 << 27) + 9,
         n - period - 1, n - 17, n - 2, n - 1],
        g.integers(0, n, size=200)]).astype(np.int64))
    x = workload.activations_bf16(2, k, 83)
    xd = upload_bits(x)
    y_ref = oracle.linear_ref(x, packed, scales, t, cols % period)
    bnd = oracle.bound(x, packed, scales, t, cols % period)
    idx = torch.from_numpy(cols).to(DEV)
    row0 = None
    for m in (1, 2):
        st, y = _launch(xd, wp, sc, t, m, n, k)
        assert st == nv.OK, st
        ys = y.index_select(1, idx)
        viol = oracle.max_violation(to_f64(ys), y_ref[:m], bnd[:m], "bf16")
        print(f"[parity] N=2^28 K=256 M={m} sampled {cols.size} columns max err/tol = {viol:.3g}", flush=True)
        assert viol <= 1.0, viol
        if row0 is None:
            row0 = bits(ys)[:1].clone()
        assert torch.equal(bits(ys)[:1], row0)
        del y, ys
    del wp, sc
    torch.cuda.empty_cache()


def test_smallest_shapes_every_kernel():
    # One output column (15 of the 16 MFMA columns past N) with the smallest
    # K (256) and with K = 4096 (every kernel can run it), at every M: all
    # kernels give the same bits, row r's bits do not depend on M, and the
    # values are within the oracle's tolerance.
    for k in (256, 4096):
        packed, scales = workload.random_codes(1, k, 90 + k)
        w = Weight(packed, scales, 0.25)
        x = workload.activations_bf16(32, k, 91 + k)
        xd = upload_bits(x)
        full = None
        for m in range(32, 0, -1):
            outs = {}
            for kernel in (nv.KERNEL_AUTO, nv.KERNEL_TILE, nv.KERNEL_PERSISTENT, nv.KERNEL_SPLIT,
                           nv.KERNEL_GENERIC, nv.KERNEL_WHOLE):
                st, y = _launch(xd, w.wp, w.sc, w.t, m, 1, k, nv.table_tile(1, k).replace(kernel=kernel),
                                out_dtype=torch.float32)
                if st == nv.ERR_TILE:
                    continue
                assert st == nv.OK, (k, m, kernel, st)
                outs[kernel] = y
            assert {nv.KERNEL_AUTO, nv.KERNEL_GENERIC} <= set(outs), (k, m, sorted(outs))
            if k == 4096 and m <= 3:
                assert {nv.KERNEL_TILE, nv.KERNEL_PERSISTENT, nv.KERNEL_SPLIT} <= set(outs), (m, sorted(outs))
            ref = bits(outs[nv.KERNEL_AUTO])
            for kernel, y in outs.items():
                assert torch.equal(bits(y), ref), f"K={k} M={m} kernel {kernel}"
            if full is None:
                full = ref.clone()
                check_parity(outs[nv.KERNEL_AUTO], x, w, label=f"N=1 K={k}")
            assert torch.equal(ref, full[:m]), f"K={k}: rows at M={m} differ from M=32"
