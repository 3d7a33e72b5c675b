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
