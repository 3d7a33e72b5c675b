"""nvfp4_linear_noalloc, the entry point for callers that cannot allocate:
its output is bit-identical to nvfp4_linear's on two calls in a row (the
second smaller), through the shapes whose exchange uses the fixed scratch
array, and it refuses a call whose exchange would not fit (gpu)."""
import numpy as np
import pytest
import torch

import verify_nvfp4_w4a16_amd as nv
import workload
from tests._gpu import DEV, Weight, bits, check_parity, upload_bits

pytestmark = pytest.mark.gpu


def _both(w, x, out_dtype=torch.bfloat16):
    m = x.shape[0]
    y_ref = torch.empty((m, w.n), dtype=out_dtype, device=DEV)
    y_na = torch.full((m, w.n), float("nan"), dtype=out_dtype, device=DEV)
    dt = nv.OUT_F32 if out_dtype == torch.float32 else nv.OUT_BF16
    s = torch.cuda.current_stream().cuda_stream
    assert nv.linear_raw(x.data_ptr(), w.wp.data_ptr(), w.sc.data_ptr(), w.t, y_ref.data_ptr(),
                         m, w.n, w.k, dt, s) == nv.OK
    st = nv.linear_noalloc_raw(x.data_ptr(), w.wp.data_ptr(), w.sc.data_ptr(), w.t, y_na.data_ptr(),
                               m, w.n, w.k, dt, s)
    torch.cuda.synchronize()
    return st, y_ref, y_na


def test_noalloc_matches_linear_two_calls_second_smaller():
    # 4096 x 12288 at 32 rows exchanges through the scratch (split 4, 64
    # column groups of 64), then 8192 x 4096 at 17 rows (split 4): each
    # output bit-equal to nvfp4_linear's, the first also within the oracle's
    # tolerance on sampled columns.
    big = Weight.from_f32(workload.weights_f32(4096, 12288, 501))
    small = Weight.from_f32(workload.weights_f32(8192, 4096, 502))
    assert nv.table_tile(4096, 12288).split > 1 and nv.table_tile(8192, 4096).split > 1
    xb = workload.activations_bf16(32, 12288, 503)
    st, y_ref, y_na = _both(big, upload_bits(xb))
    assert st == nv.OK
    assert torch.equal(bits(y_na), bits(y_ref))
    cols = np.unique(np.concatenate([np.arange(32), workload.rng(504).integers(0, 4096, 256)]))
    check_parity(y_na, xb, big, cols=cols, label="noalloc 4096x12288 M=32")
    xs = workload.activations_bf16(17, 4096, 505)
    st, y_ref, y_na = _both(small, upload_bits(xs))
    assert st == nv.OK
    assert torch.equal(bits(y_na), bits(y_ref))
    # and the one-row path, which needs no exchange
    st, y_ref, y_na = _both(small, upload_bits(xs[:1]), torch.float32)
    assert st == nv.OK and torch.equal(bits(y_na), bits(y_ref))
    assert not nv.timeout_status()


def test_noalloc_refuses_an_exchange_beyond_the_scratch():
    # 6144 x 4096 at 32 rows (split 8, 48 column groups of 128) would
    # exchange 48 x 224 KiB, more than the 8 MiB of scratch: refused before
    # anything is launched (y keeps its canary), while nvfp4_linear, with its
    # own workspace, runs it.
    w = Weight.from_f32(workload.weights_f32(6144, 4096, 506))
    assert nv.table_tile(6144, 4096).split == 8
    x = upload_bits(workload.activations_bf16(32, 4096, 507))
    st, y_ref, y_na = _both(w, x, torch.float32)
    assert st == nv.ERR_SCRATCH
    assert torch.isnan(y_na).all() and not torch.isnan(y_ref).any()
    # at 16 rows the same product fits (four wavefronts per workgroup)
    x16 = upload_bits(workload.activations_bf16(16, 4096, 508))
    st, y_ref, y_na = _both(w, x16)
    assert st == nv.OK and torch.equal(bits(y_na), bits(y_ref))
