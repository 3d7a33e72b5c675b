"""Launch behaviour on the GPU: determinism, graph replay, out-of-bounds
guards, M = 0, and errors from the binding (gpu)."""
import numpy as np
import pytest
import torch

import verify_nvfp4_w4a16_amd as nv
import workload
from tests._gpu import DEV, Weight, bits, run, upload_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def weight():
    return Weight.from_f32(workload.weights_f32(3000, 2048, 91))


def test_init_reports_gfx950():
    nv.init()


def test_launch_info_names_the_dispatched_kernel():
    # The per-tile kernel at one row, the many-row kernel at 16 and 32 rows on
    # the decode round's shapes; the trace name carries the template
    # arguments (column tiles, row tiles, buffers or wavefronts, output type,
    # several-product launch).
    for n, k in ((8192, 4096), (4096, 8192), (24576, 4096), (4096, 12288)):
        assert nv.kernel_name(1, n, k).startswith("nvfp4_skinny_tile<1, 1, ")
        assert nv.kernel_name(16, n, k).startswith("nvfp4_skinny_split<1, 1, ")
        assert nv.kernel_name(32, n, k).startswith("nvfp4_skinny_split<1, 2, ")
        assert nv.kernel_name(32, n, k).endswith(", false, false>")
    assert nv.kernel_name(1, 151552, 4096, nv.OUT_F32).endswith(", true, false>")
    assert nv.launch_info(0, 8192, 4096) == "none"
    info = nv.launch_info(32, 8192, 4096)
    assert " grid=" in info and " block=" in info and " parts=4" in info


def test_read_probe_reads_and_leaves_the_sink():
    a = torch.zeros(1 << 20, dtype=torch.uint8, device=DEV)
    b = torch.zeros(4096, dtype=torch.uint8, device=DEV)
    sink = torch.full((1,), 7, dtype=torch.int32, device=DEV)
    st = nv.read_probe_raw(a.data_ptr(), a.numel(), b.data_ptr(), b.numel(), sink.data_ptr(),
                           torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == nv.OK and int(sink.item()) == 7


def test_deterministic(weight):
    x = workload.activations_bf16(23, 2048, 92)
    a = bits(run(x, weight)).clone()
    for _ in range(3):
        assert torch.equal(bits(run(x, weight)), a)


def test_canary_guards_and_untouched_rows(weight):
    m, n, k = 5, weight.n, weight.k
    x = upload_bits(workload.activations_bf16(m, k, 93))
    for dtype, fill in ((torch.bfloat16, -12345), (torch.float32, -12345678)):
        # y sits inside a larger buffer whose other elements are guards
        flat = torch.empty((34 * n + 64,), dtype=dtype, device=DEV)
        bits(flat).fill_(fill)
        y = flat[32:32 + m * n].view(m, n)
        out = nv.linear(x, weight.wp, weight.sc, weight.t, out=y)
        torch.cuda.synchronize()
        fb = bits(flat)
        assert (fb[:32] == fill).all() and (fb[32 + m * n:] == fill).all()
        assert not (bits(out) == fill).all()


def test_m_zero_launches_nothing(weight):
    x = torch.empty((0, weight.k), dtype=torch.bfloat16, device=DEV)
    y = torch.empty((0, weight.n), dtype=torch.bfloat16, device=DEV)
    nv.linear(x, weight.wp, weight.sc, weight.t, out=y)
    torch.cuda.synchronize()


def test_graph_replay_matches_eager(weight):
    xs = [upload_bits(workload.activations_bf16(m, weight.k, 94 + m)) for m in (1, 16, 32)]
    ys = [torch.empty((x.shape[0], weight.n), dtype=torch.bfloat16, device=DEV) for x in xs]
    eager = []
    for x in xs:
        eager.append(bits(nv.linear(x, weight.wp, weight.sc, weight.t)).clone())
    nv.init()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for x, y in zip(xs, ys):
                nv.linear(x, weight.wp, weight.sc, weight.t, out=y)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(4):
        for y in ys:
            y.zero_()
        g.replay()
        torch.cuda.synchronize()
        for y, e in zip(ys, eager):
            assert torch.equal(bits(y), e), f"replay {rep} differs from eager"
        # eager work between replays
        run(workload.activations_bf16(3, weight.k, 99), weight)


def test_binding_rejects_bad_arguments(weight):
    x = torch.zeros((33, weight.k), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(nv.Nvfp4Error) as e:
        nv.linear(x, weight.wp, weight.sc, weight.t)
    assert e.value.status == nv.ERR_SHAPE
    with pytest.raises(TypeError):
        nv.linear(x[:2].float(), weight.wp, weight.sc, weight.t)
    with pytest.raises(ValueError):
        nv.linear(x[:2], weight.wp[:, :-16], weight.sc, weight.t)


def test_subnormal_inputs_and_products_recorded():
    # bf16 subnormal activations and fp32-subnormal products: measured on
    # MI355X, the bf16 MFMA keeps both exactly (no flush to zero); this pins
    # that, and that every kernel and every row count give the same bits.
    n, k = 16, 4096
    packed = np.zeros((n, k // 2), dtype=np.uint8)
    scales = np.full((n, k // 16), 0x38, dtype=np.uint8)
    packed[3, 5 // 2] = 0x7 << 4            # (n=3, k=5): code 7 = 6.0, high nibble (odd k)
    scales[3, 0] = 0x7E                      # 448: Wd[3, 5] = 2688
    packed[4, 7 // 2] = 0x1 << 4             # (n=4, k=7): code 1 = 0.5
    scales[4, 0] = 0x01                      # 2^-9: Wd[4, 7] = 2^-10
    w = Weight(packed, scales, 1.0)
    x = np.zeros((2, k), dtype=np.uint16)
    x[0, 5] = 0x0008                         # 2^-130, a bf16 subnormal
    x[0, 7] = 0x0080                         # 2^-126, the smallest normal bf16
    x[1, 5] = 0x0080
    x[1, 7] = 0x3F80                         # 1.0
    y = run(x, w, torch.float32).cpu().numpy().astype(np.float64)
    assert y[1, 3] == 2688.0 * 2.0 ** -126 and y[1, 4] == 2.0 ** -10
    sub_x, sub_p = y[0, 3], y[0, 4]
    assert sub_x in (0.0, 2688.0 * 2.0 ** -130), sub_x
    assert sub_p in (0.0, 2.0 ** -136), sub_p
    print(f"[subnormal] bf16 subnormal x: {'kept' if sub_x else 'flushed'}; "
          f"fp32-subnormal product: {'kept' if sub_p else 'flushed'}", flush=True)
    assert sub_x and sub_p
    assert not np.delete(y, [3, 4], axis=1).any()
    # same bits for one row alone and through every kernel
    ref = bits(run(x, w, torch.float32)).clone()
    assert torch.equal(bits(run(x[:1], w, torch.float32)), ref[:1])
    xt = upload_bits(x)
    for kernel in (nv.KERNEL_PERSISTENT, nv.KERNEL_TILE, nv.KERNEL_SPLIT, nv.KERNEL_GENERIC, nv.KERNEL_WHOLE):
        yk = torch.empty((2, n), dtype=torch.float32, device=DEV)
        st = nv.linear_tiled_raw(xt.data_ptr(), w.wp.data_ptr(), w.sc.data_ptr(), w.t, yk.data_ptr(), 2, n, k,
                                 nv.OUT_F32, nv.table_tile(n, k).replace(kernel=kernel),
                                 torch.cuda.current_stream().cuda_stream)
        if st == nv.ERR_TILE:
            continue
        assert st == nv.OK
        torch.cuda.synchronize()
        assert torch.equal(bits(yk), ref), kernel


_TIMEOUT_CHILD = r"""
import numpy as np, torch
import verify_nvfp4_w4a16_amd as nv
import workload
n, k = 4096, 8192                          # split > 1: the many-row kernel's parts meet through flags
w = workload.weights_f32(n, k, 5)
packed, scales, t = nv.pack(w)
dev = torch.device("cuda:0")
wp, sc = torch.from_numpy(packed).to(dev), torch.from_numpy(scales).to(dev)
assert nv.table_tile(n, k).split > 1
assert not nv.timeout_status()
for m, expect_nan in ((17, True), (32, True), (1, False)):
    xb = workload.activations_bf16(m, k, 6 + m)
    x = torch.from_numpy(xb.view(np.int16)).to(dev).view(torch.bfloat16)
    y = nv.linear(x, wp, sc, t, out_dtype=torch.float32)
    torch.cuda.synchronize()
    nan = torch.isnan(y)
    assert bool(nan.all()) if expect_nan else not bool(nan.any()), (m, int(nan.sum()))
    # the host sees the time-out through the status word, which reading clears
    assert nv.timeout_status() == expect_nan, m
    assert not nv.timeout_status()
# the FP8 product's many-row form meets through the same exchange (4096
# columns: groups in separate workgroups); one row takes the register path
codes, fscales = nv.fp8_pack(workload.weights_f32(n, k, 7))
wd, sd = torch.from_numpy(codes).to(dev), torch.from_numpy(fscales).to(dev)
for m, expect_nan in ((16, True), (1, False)):
    xb = workload.activations_bf16(m, k, 60 + m)
    x = torch.from_numpy(xb.view(np.int16)).to(dev).view(torch.bfloat16)
    y = torch.empty((m, n), dtype=torch.float32, device=dev)
    st = nv.fp8_linear_raw(x.data_ptr(), wd.data_ptr(), sd.data_ptr(), y.data_ptr(), m, n, k, nv.OUT_F32,
                           torch.cuda.current_stream().cuda_stream)
    assert st == nv.OK, st
    torch.cuda.synchronize()
    nan = torch.isnan(y)
    assert bool(nan.all()) if expect_nan else not bool(nan.any()), ("fp8", m, int(nan.sum()))
    assert nv.timeout_status() == expect_nan, ("fp8", m)
print("timeout path ok", flush=True)
"""

_LATE_PRODUCER_CHILD = r"""
import numpy as np, torch
import verify_nvfp4_w4a16_amd as nv
import workload
# NVFP4_TEST_SPLIT_TIMEOUT=2: producers set their flags only long after their
# consumer gave up.  A replayed graph reuses every launch argument, so the
# next replay must not take those late flags (and the sums behind them) for
# its own: every replay, with new x each time, must give NaN everywhere.
n, k, m = 4096, 8192, 17
w = workload.weights_f32(n, k, 5)
packed, scales, t = nv.pack(w)
dev = torch.device("cuda:0")
wp, sc = torch.from_numpy(packed).to(dev), torch.from_numpy(scales).to(dev)
assert nv.table_tile(n, k).split > 1
nv.init()
x = torch.empty((m, k), dtype=torch.bfloat16, device=dev)
y = torch.empty((m, n), dtype=torch.float32, device=dev)
s = torch.cuda.Stream()
s.wait_stream(torch.cuda.current_stream())
g = torch.cuda.CUDAGraph()
with torch.cuda.stream(s):
    with torch.cuda.graph(g, stream=s):
        nv.linear(x, wp, sc, t, out=y)
torch.cuda.current_stream().wait_stream(s)
torch.cuda.synchronize()
for rep in range(4):
    xb = workload.activations_bf16(m, k, 40 + rep)
    x.copy_(torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16))
    y.fill_(0.0)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    finite = int(torch.isfinite(y).sum())
    print(f"replay {rep}: finite outputs {finite}", flush=True)
    assert finite == 0, (rep, finite)
    assert nv.timeout_status()
print("late producers ok", flush=True)
"""


def _run_child(code, mode):
    import os, subprocess, sys
    env = dict(os.environ, NVFP4_TEST_SPLIT_TIMEOUT=mode)
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env["PYTHONPATH"] = root + os.pathsep + os.path.join(root, "tests") + os.pathsep + env.get("PYTHONPATH", "")
    r = subprocess.run([sys.executable, "-c", code], env=env, cwd=root, capture_output=True, text=True,
                       timeout=300)
    print(r.stdout[-2000:], r.stderr[-2000:], flush=True)
    return r


def test_replay_after_time_out_never_takes_late_flags():
    # The generation word of a column group advances with every call, so a
    # flag stored late by a timed-out call's producer never matches what a
    # later call (here: the next replay of the same captured graph) waits for.
    r = _run_child(_LATE_PRODUCER_CHILD, "2")
    assert r.returncode == 0 and "late producers ok" in r.stdout



def test_many_row_time_out_writes_nan():
    # NVFP4_TEST_SPLIT_TIMEOUT=1 (read once per process): the producers of the
    # many-row kernel set no flags and the consumers give up after a few
    # polls; every output of the product must then be NaN rather than a
    # hang or a partial sum.  The per-tile kernel (M = 1) has no exchange.
    r = _run_child(_TIMEOUT_CHILD, "1")
    assert r.returncode == 0 and "timeout path ok" in r.stdout
