"""Decode-round benchmark of the NVFP4 W4A16 skinny product on one MI355X.

Workload: 48 layers x {(8192,4096), (4096,8192), (24576,4096), (4096,12288)}
NVFP4 weights (10,468,982,784 weights; 5,888,802,816 bytes of packed nibbles
plus e4m3 scales), weights N(0, 0.02) packed by nvfp4_pack, bf16 N(0,1)
activations drawn per (layer, projection, M).  One step runs the whole round
back-to-back on one stream at each M in {1, 16, 32}, each round replayed from
one captured HIP graph of 192 nvfp4_linear launches.

value: weight-stream GB/s = packed + scale bytes of every timed product over
the timed wall time (decimal GB/s), all three M together; per-M figures and %
of the 8.0 TB/s MI355X peak are in "per_m".  After the timed steps (outside
the timed region) the benchmark also measures, each from graphs of its own:
every kernel of the round on its own launches (the roofline is the kernel
with the most GPU time per round), a plain read of the round's bytes (the
ceiling of 192 separate launches), and the other workloads of the product
(one 1024 x 1024 linear, the 4096 x 4096 product at M = 1..32, the
12288 x 4096 QKV-style product at M = 16..32, the 151552 x 4096 output head
at M = 1..32), each over weight copies rotated through more than 512 MB so
every launch reads HBM.  Prints one JSON line on stdout.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workload  # noqa: E402

PEAK_HBM_GBPS = 8000.0
PEAK_BF16_MFMA_TFLOPS = 2500.0
BYTES_PER_WEIGHT = 0.5625          # 4-bit code + one e4m3 byte per 16 weights
CPU_BASELINE_MIN_S = 10.0           # the oracle runs products until this much CPU time has passed ...
CPU_BASELINE_MAX_S = 30.0           # ... and stops starting new ones past this
CPU_BASELINE_LAYERS = 32            # layers whose packed bytes stay on the host for it
COLD_BYTES = 512 << 20              # weight copies rotated per timed launch sequence
KERNEL_SOURCES = [os.path.join(ROOT, "verify_nvfp4_w4a16_amd", "csrc", "kernels", f)
                  for f in ("nvfp4_common.h", "nvfp4_linear.hip", "nvfp4_gemm.hip", "nvfp4_fused.hip", "w8a16.hip")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_decode_round.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_cores() -> int:
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:
        return max(1, min(16, os.cpu_count() or 1))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def kernel_source_hash() -> str:
    """SHA-256 prefix of the kernel sources with comment and blank lines
    removed, so a counter profile stays attached to the code it measured
    across comment-only edits."""
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, encoding="utf-8") as f:
            code = [ln.rstrip() for ln in f if ln.strip() and not ln.lstrip().startswith("//")]
        h.update("\n".join(code).encode())
    return h.hexdigest()[:16]


WARM_MS = 20.0      # replay at least this long before timing: a graph timed right after a pause ran up to 10 % slow


def timed_graph(torch, stream, fn, reps: int = 5, warm: int = 2) -> float:
    """Median milliseconds of one replay of a graph capturing fn(stream_handle),
    after at least `warm` replays and WARM_MS of them."""
    g = torch.cuda.CUDAGraph()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            fn(stream.cuda_stream)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    ts = []
    with torch.cuda.stream(stream):
        s0, e0 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record(stream)
        g.replay()
        e0.record(stream)
        e0.synchronize()
        warm = max(warm, min(200, int(WARM_MS / max(s0.elapsed_time(e0), 1e-3))))
        for i in range(warm + reps):
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record(stream)
            g.replay()
            e.record(stream)
            e.synchronize()
            if i >= warm:
                ts.append(s.elapsed_time(e))
    del g
    return float(np.median(ts))


class Round:
    """The 192 packed weights of the decode round, resident in HBM."""

    def __init__(self, torch, dev, layers: int):
        import verify_nvfp4_w4a16_amd as nv
        self.layers = layers
        self.items = []           # (layer, proj, shape, wp, sc, t)
        self.host = {}            # (layer, proj) -> (packed, scales, t) of the CPU-baseline layers
        jobs = [(l, p) for l in range(layers) for p in range(len(workload.ROUND_SHAPES))]

        def gen(job):
            l, p = job
            s = workload.ROUND_SHAPES[p]
            return job, workload.weights_f32(s.n, s.k, workload.round_weight_seed(l, p))

        t0 = time.time()
        with ThreadPoolExecutor(max(1, cpu_cores() // 2)) as ex:
            for (l, p), w in ex.map(gen, jobs):
                packed, scales, t = nv.pack(w)
                del w
                wp = torch.from_numpy(packed).to(dev, non_blocking=False)
                sc = torch.from_numpy(scales).to(dev, non_blocking=False)
                if l < CPU_BASELINE_LAYERS:
                    self.host[(l, p)] = (packed, scales, t)
                self.items.append((l, p, workload.ROUND_SHAPES[p], wp, sc, t))
        torch.cuda.synchronize()
        log(f"[bench] packed and uploaded {len(self.items)} weights in {time.time() - t0:.1f}s")

    def weight_bytes(self) -> int:
        return sum(s.n * s.k // 2 + s.n * s.k // 16 for _, _, s, _, _, _ in self.items)

    def algorithmic_bytes(self, m: int) -> int:
        """Weights + x read once + bf16 y written once."""
        return self.weight_bytes() + sum(2 * m * s.k + 2 * m * s.n for _, _, s, _, _, _ in self.items)


class Launches:
    """Activations and outputs of one round at row count m."""

    def __init__(self, torch, dev, rnd: Round, m: int):
        import verify_nvfp4_w4a16_amd as nv
        self.nv, self.m = nv, m
        self.calls = []
        self.ys = {}
        for l, p, s, wp, sc, t in rnd.items:
            xb = workload.activations_bf16(m, s.k, workload.round_act_seed(l, p, m))
            x = torch.from_numpy(xb.view(np.int16)).to(dev).view(torch.bfloat16)
            if p not in self.ys:
                self.ys[p] = torch.empty((m, s.n), dtype=torch.bfloat16, device=dev)
            y = self.ys[p]
            self.calls.append((x.data_ptr(), wp.data_ptr(), sc.data_ptr(), t, y.data_ptr(),
                               m, s.n, s.k, x))

    def launch(self, stream_handle: int, which=None) -> None:
        nv = self.nv
        for i, (xp, wpp, scp, t, yp, m, n, k, _) in enumerate(self.calls):
            if which is not None and i not in which:
                continue
            st = nv.linear_raw(xp, wpp, scp, t, yp, m, n, k, nv.OUT_BF16, stream_handle)
            if st != nv.OK:
                raise nv.Nvfp4Error(st, "nvfp4_linear")


def copy_bandwidth(torch, dev) -> float:
    a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(10):
        b.copy_(a)
    e.record()
    e.synchronize()
    ms = s.elapsed_time(e) / 10
    del a, b
    return 2 * (1 << 30) / (ms * 1e-3) / 1e9


def per_kernel(torch, stream, rnd: Round, launches: dict, ms_list) -> list:
    """Every kernel of the round at each timed M, timed on its own launches
    (a graph of those launches in round order, HIP events on its stream)."""
    nv = launches[ms_list[0]].nv
    rows = []
    for m in ms_list:
        groups = {}
        for i, (_, _, s, _, _, _) in enumerate(rnd.items):
            groups.setdefault(nv.kernel_name(m, s.n, s.k), []).append(i)
        lc = launches[m]
        for name, idx in groups.items():
            which = set(idx)
            ms = timed_graph(torch, stream, lambda h: lc.launch(h, which))
            avg_us = ms * 1e3 / len(idx)
            shapes = sorted({(rnd.items[i][2].n, rnd.items[i][2].k) for i in idx})
            wbytes = sum(rnd.items[i][2].n * rnd.items[i][2].k * BYTES_PER_WEIGHT for i in idx) / len(idx)
            xy = sum(2 * m * (rnd.items[i][2].n + rnd.items[i][2].k) for i in idx) / len(idx)
            flops = sum(2.0 * m * rnd.items[i][2].n * rnd.items[i][2].k for i in idx) / len(idx)
            rows.append({"m": m, "kernel": name, "launches_per_round": len(idx),
                         "shapes": [f"{n}x{k}" for n, k in shapes],
                         "avg_launch_us": avg_us, "round_share_us": avg_us * len(idx),
                         "weight_bytes_per_launch": wbytes, "xy_bytes_per_launch": xy,
                         "weight_GBps": wbytes / (avg_us * 1e-6) / 1e9,
                         "frac_of_peak": wbytes / (avg_us * 1e-6) / 1e9 / PEAK_HBM_GBPS,
                         "mfma_TFLOPs": flops / (avg_us * 1e-6) / 1e12})
    return rows


def read_ceiling(torch, stream, rnd: Round) -> dict:
    """A plain read of each product's packed weights and scales, one launch per
    product in round order: the round ceiling of separate launches, and per
    shape the time of one read (cold: the round is 5.9 GB)."""
    import verify_nvfp4_w4a16_amd as nv
    sink = torch.zeros(64, dtype=torch.int32, device=rnd.items[0][3].device)

    def run(h, which=None):
        for i, (_, _, s, wp, sc, _) in enumerate(rnd.items):
            if which is not None and i not in which:
                continue
            st = nv.read_probe_raw(wp.data_ptr(), wp.numel(), sc.data_ptr(), sc.numel(), sink.data_ptr(), h)
            if st != nv.OK:
                raise nv.Nvfp4Error(st, "nvfp4_read_probe")

    ms = timed_graph(torch, stream, run)
    out = {"round_ms": ms, "round_GBps": rnd.weight_bytes() / (ms * 1e-3) / 1e9, "per_shape_us": {}}
    for p, s in enumerate(workload.ROUND_SHAPES):
        which = {i for i, it in enumerate(rnd.items) if it[1] == p}
        ms_p = timed_graph(torch, stream, lambda h: run(h, which))
        us = ms_p * 1e3 / len(which)
        out["per_shape_us"][f"{s.n}x{s.k}"] = {"us": us, "GBps": s.n * s.k * BYTES_PER_WEIGHT / (us * 1e-6) / 1e9}
    return out


def config_timings(torch, dev, stream) -> dict:
    """The product's other workloads, each over weight copies rotated through
    more than 512 MB (distinct addresses, so every launch reads HBM)."""
    import verify_nvfp4_w4a16_amd as nv
    out = {}

    def copies(shape, seed):
        packed, scales, t = nv.pack(workload.weights_f32(shape.n, shape.k, seed))
        wp0, sc0 = torch.from_numpy(packed).to(dev), torch.from_numpy(scales).to(dev)
        wbytes = packed.nbytes + scales.nbytes
        count = max(2, -(-COLD_BYTES // wbytes))
        return [(wp0.clone(), sc0.clone()) for _ in range(count)], t, wbytes

    def timing(ws, t, n, k, x, y, dtype):
        def run(h):
            for wp, sc in ws:
                st = nv.linear_raw(x.data_ptr(), wp.data_ptr(), sc.data_ptr(), t, y.data_ptr(), x.shape[0], n, k,
                                   dtype, h)
                if st != nv.OK:
                    raise nv.Nvfp4Error(st, "nvfp4_linear")
        return timed_graph(torch, stream, run) * 1e3 / len(ws)

    def xs(m, k, seed, outliers=False):
        xb = workload.activations_bf16(m, k, seed, outliers=outliers)
        return torch.from_numpy(xb.view(np.int16)).to(dev).view(torch.bfloat16)

    s = workload.SINGLE
    ws, t, wb = copies(s, workload.SEEDS["single"][0])
    x = xs(1, s.k, workload.SEEDS["single"][1])
    y = torch.empty((1, s.n), dtype=torch.bfloat16, device=dev)
    us = timing(ws, t, s.n, s.k, x, y, nv.OUT_BF16)
    out["single_1024x1024_M1"] = {"us_per_launch": us, "weight_GBps": wb / (us * 1e-6) / 1e9, "copies": len(ws),
                                  "kernel": nv.kernel_name(1, s.n, s.k),
                                  "note": "launch-latency bound (0.59 MB): the GB/s is not a bandwidth figure"}
    del ws

    s = workload.INVARIANCE
    ws, t, wb = copies(s, workload.SEEDS["invariance"][0])
    xfull = xs(32, s.k, workload.SEEDS["invariance"][1])
    per = {}
    for m in range(1, 33):
        y = torch.empty((m, s.n), dtype=torch.bfloat16, device=dev)
        us = timing(ws, t, s.n, s.k, xfull[:m], y, nv.OUT_BF16)
        per[str(m)] = {"us": us, "weight_GBps": wb / (us * 1e-6) / 1e9, "kernel": nv.kernel_name(m, s.n, s.k)}
    out["invariance_4096x4096_M1to32"] = {"copies": len(ws), "per_m": per}
    del ws

    s = workload.QKV
    ws, t, wb = copies(s, workload.SEEDS["qkv"][0])
    xfull = xs(32, s.k, workload.SEEDS["qkv"][1], outliers=True)
    per = {}
    for m in range(16, 33):
        y = torch.empty((m, s.n), dtype=torch.bfloat16, device=dev)
        us = timing(ws, t, s.n, s.k, xfull[:m], y, nv.OUT_BF16)
        per[str(m)] = {"us": us, "weight_GBps": wb / (us * 1e-6) / 1e9, "kernel": nv.kernel_name(m, s.n, s.k)}
    out["qkv_12288x4096_M16to32"] = {"copies": len(ws), "per_m": per,
                                     "step_17_over_16": per["17"]["us"] / per["16"]["us"]}
    del ws

    s = workload.HEAD
    ws, t, wb = copies(s, workload.SEEDS["head"][0])
    xfull = xs(32, s.k, workload.SEEDS["head"][1])
    per = {}
    for m in range(1, 33):
        y = torch.empty((m, s.n), dtype=torch.float32, device=dev)
        us = timing(ws, t, s.n, s.k, xfull[:m], y, nv.OUT_F32)
        per[str(m)] = {"us": us, "weight_GBps": wb / (us * 1e-6) / 1e9,
                       "kernel": nv.kernel_name(m, s.n, s.k, nv.OUT_F32)}
    out["head_151552x4096_fp32_M1to32"] = {"copies": len(ws), "per_m": per}
    del ws
    torch.cuda.synchronize()
    return out


def next_rows(torch, dev, stream) -> dict:
    """The other regimes and forms of the product, timed cold like the
    workloads above: the many-row GEMM (M = 64, 256, 1024) and the expand path
    (M = 4096) on the decode round's shapes, the fused forms (two projections
    over one x, the silu(gate) * up input, de-interleaved Q|K|V|Z output, a
    grouped launch over 128 experts) and the FP8 block-scaled product."""
    import verify_nvfp4_w4a16_amd as nv
    out = {}
    def rotate(make, nbytes):
        return [make() for _ in range(max(2, -(-COLD_BYTES // nbytes)))]

    def xs(m, k, seed):
        xb = workload.activations_bf16(m, k, seed)
        return torch.from_numpy(xb.view(np.int16)).to(dev).view(torch.bfloat16)

    def nvfp4_weight(n, k, seed):
        packed, scales, t = nv.pack(workload.weights_f32(n, k, seed))
        return torch.from_numpy(packed).to(dev), torch.from_numpy(scales).to(dev), t, packed.nbytes + scales.nbytes

    def call(fn, *args):
        st = fn(*args)
        if st != nv.OK:
            raise nv.Nvfp4Error(st, getattr(fn, "__name__", "call"))

    gemm = {}
    for s in workload.ROUND_SHAPES:
        wp0, sc0, t, wb = nvfp4_weight(s.n, s.k, 7)
        ws = rotate(lambda: (wp0.clone(), sc0.clone()), wb)
        for m in (64, 256, 1024):
            x = xs(m, s.k, 8)
            y = torch.empty((m, s.n), dtype=torch.bfloat16, device=dev)
            def run(h):
                for wp, sc in ws:
                    call(nv.gemm_raw, x.data_ptr(), wp.data_ptr(), sc.data_ptr(), t, y.data_ptr(), m, s.n, s.k,
                         nv.OUT_BF16, h)
            us = timed_graph(torch, stream, run) * 1e3 / len(ws)
            def run_mm(h):
                for wp, sc in ws:
                    call(nv.matmul_raw, x.data_ptr(), wp.data_ptr(), sc.data_ptr(), t, y.data_ptr(), m, s.n, s.k,
                         nv.OUT_BF16, h)
            us_mm = timed_graph(torch, stream, run_mm) * 1e3 / len(ws)
            tf = 2.0 * m * s.n * s.k / (us * 1e-6) / 1e12
            gemm[f"{s.n}x{s.k}_M{m}"] = {"us": us, "TFLOPs": tf, "frac_of_bf16_mfma_peak": tf / PEAK_BF16_MFMA_TFLOPS,
                                        "weight_GBps": wb / (us * 1e-6) / 1e9, "matmul_dispatch_us": us_mm}
        del ws
    out["gemm_regime"] = gemm

    n, k, m = 8192, 4096, 4096
    wp0, sc0, t, wb = nvfp4_weight(n, k, 9)
    x = xs(m, k, 10)
    y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    wbf = torch.empty((n, k), dtype=torch.bfloat16, device=dev)
    # one graph of REPS calls per figure, so a graph launch's own latency is
    # spread over them (these rows reuse one weight: warm caches)
    REPS = 5

    def per_call(fn):
        return timed_graph(torch, stream, lambda h: [fn(h) for _ in range(REPS)]) * 1e3 / REPS

    us_expand = per_call(lambda h: call(nv.dequant_bf16_raw, wp0.data_ptr(), sc0.data_ptr(), t, 0,
                                        wbf.data_ptr(), n, k, h))
    us_exp_gemm = per_call(lambda h: call(nv.gemm_expanded_raw, x.data_ptr(), wbf.data_ptr(), t,
                                          y.data_ptr(), m, n, k, nv.OUT_BF16, h))
    us_gemm = per_call(lambda h: call(nv.gemm_raw, x.data_ptr(), wp0.data_ptr(), sc0.data_ptr(), t,
                                      y.data_ptr(), m, n, k, nv.OUT_BF16, h))
    # the library GEMM: its first call (handle, workspace, plan) outside capture
    call(nv.gemm_library_raw, x.data_ptr(), wbf.data_ptr(), t, y.data_ptr(), m, n, k, nv.OUT_BF16,
         stream.cuda_stream)
    torch.cuda.synchronize()
    us_lib = per_call(lambda h: call(nv.gemm_library_raw, x.data_ptr(), wbf.data_ptr(), t,
                                     y.data_ptr(), m, n, k, nv.OUT_BF16, h))
    # the pages' third regime done per call: expand, then the library GEMM
    def expand_then_library(h):
        call(nv.dequant_bf16_raw, wp0.data_ptr(), sc0.data_ptr(), t, 0, wbf.data_ptr(), n, k, h)
        call(nv.gemm_library_raw, x.data_ptr(), wbf.data_ptr(), t, y.data_ptr(), m, n, k, nv.OUT_BF16, h)
    us_exp_lib = per_call(expand_then_library)
    out["expand_8192x4096_M4096"] = {"expand_us": us_expand, "expand_GBps_read_plus_write":
                                     (wb + 2 * n * k) / (us_expand * 1e-6) / 1e9,
                                     "gemm_expanded_us": us_exp_gemm, "gemm_nvfp4_us": us_gemm,
                                     "gemm_expanded_TFLOPs": 2.0 * m * n * k / (us_exp_gemm * 1e-6) / 1e12,
                                     "gemm_library_us": us_lib,
                                     "gemm_library_TFLOPs": 2.0 * m * n * k / (us_lib * 1e-6) / 1e12,
                                     "expand_then_library_us": us_exp_lib}
    # the library GEMM on the decode round's shapes at 1024 and 4096 rows
    # against nvfp4_gemm (one weight, warm: both reread it per row tile)
    lib_rows = {}
    for s in workload.ROUND_SHAPES:
        wp1, sc1, t1, _ = nvfp4_weight(s.n, s.k, 11)
        wbf1 = torch.empty((s.n, s.k), dtype=torch.bfloat16, device=dev)
        call(nv.dequant_bf16_raw, wp1.data_ptr(), sc1.data_ptr(), t1, 0, wbf1.data_ptr(), s.n, s.k,
             stream.cuda_stream)
        for mm in (1024, 4096):
            x1 = xs(mm, s.k, 12)
            y1 = torch.empty((mm, s.n), dtype=torch.bfloat16, device=dev)
            call(nv.gemm_library_raw, x1.data_ptr(), wbf1.data_ptr(), t1, y1.data_ptr(), mm, s.n, s.k,
                 nv.OUT_BF16, stream.cuda_stream)
            torch.cuda.synchronize()
            ul = per_call(lambda h: call(nv.gemm_library_raw, x1.data_ptr(), wbf1.data_ptr(), t1,
                                         y1.data_ptr(), mm, s.n, s.k, nv.OUT_BF16, h))
            ug = per_call(lambda h: call(nv.gemm_raw, x1.data_ptr(), wp1.data_ptr(), sc1.data_ptr(), t1,
                                         y1.data_ptr(), mm, s.n, s.k, nv.OUT_BF16, h))
            def etl(h):
                call(nv.dequant_bf16_raw, wp1.data_ptr(), sc1.data_ptr(), t1, 0, wbf1.data_ptr(), s.n, s.k, h)
                call(nv.gemm_library_raw, x1.data_ptr(), wbf1.data_ptr(), t1, y1.data_ptr(), mm, s.n, s.k,
                     nv.OUT_BF16, h)
            ue = per_call(etl)
            fl = 2.0 * mm * s.n * s.k
            lib_rows[f"{s.n}x{s.k}_M{mm}"] = {"library_us": ul, "nvfp4_gemm_us": ug, "expand_then_library_us": ue,
                                               "library_TFLOPs": fl / (ul * 1e-6) / 1e12,
                                               "nvfp4_gemm_TFLOPs": fl / (ug * 1e-6) / 1e12}
        del wbf1
    out["library_gemm"] = lib_rows
    del wbf

    fused = {}
    n, k = 12288, 4096
    a = nvfp4_weight(n, k, 11)
    b = nvfp4_weight(n, k, 12)
    pairs = rotate(lambda: (a[0].clone(), a[1].clone(), b[0].clone(), b[1].clone()), 2 * a[3])
    for m in (1, 8):
        x = xs(m, k, 13)
        y0 = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        y1 = torch.empty_like(y0)
        def run(h):
            for wa, sa, wb_, sb in pairs:
                call(nv.linear_dual_raw, x.data_ptr(), wa.data_ptr(), sa.data_ptr(), a[2], y0.data_ptr(),
                     wb_.data_ptr(), sb.data_ptr(), b[2], y1.data_ptr(), m, n, k, nv.OUT_BF16, h)
        us = timed_graph(torch, stream, run) * 1e3 / len(pairs)
        fused[f"dual_2x{n}x{k}_M{m}"] = {"us": us, "weight_GBps": 2 * a[3] / (us * 1e-6) / 1e9}
    del pairs
    n, k = 4096, 12288
    wp0, sc0, t, wb = nvfp4_weight(n, k, 14)
    ws = rotate(lambda: (wp0.clone(), sc0.clone()), wb)
    for m in (1, 2):
        g, u = xs(m, k, 15), xs(m, k, 16)
        y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        def run(h):
            for wp, sc in ws:
                call(nv.linear_silu_input_raw, g.data_ptr(), u.data_ptr(), wp.data_ptr(), sc.data_ptr(), t,
                     y.data_ptr(), m, n, k, nv.OUT_BF16, h)
        us = timed_graph(torch, stream, run) * 1e3 / len(ws)
        fused[f"silu_input_{n}x{k}_M{m}"] = {"us": us, "weight_GBps": wb / (us * 1e-6) / 1e9}
    del ws
    n, k, widths = 12288, 4096, [256, 128, 128, 256]
    wp0, sc0, t, wb = nvfp4_weight(n, k, 17)
    ws = rotate(lambda: (wp0.clone(), sc0.clone()), wb)
    for m in (1, 8):
        x = xs(m, k, 18)
        y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        def run(h):
            for wp, sc in ws:
                call(nv.linear_deinterleave_raw, x.data_ptr(), wp.data_ptr(), sc.data_ptr(), t, y.data_ptr(),
                     m, n, k, nv.OUT_BF16, widths, h)
        us = timed_graph(torch, stream, run) * 1e3 / len(ws)
        fused[f"qkvz_{n}x{k}_M{m}"] = {"us": us, "weight_GBps": wb / (us * 1e-6) / 1e9}
    del ws
    experts, n, k, m = 128, 1536, 4096, 2
    wp0, sc0, t, wb = nvfp4_weight(n, k, 19)
    ews = [(wp0.clone(), sc0.clone()) for _ in range(experts)]
    xe = [xs(m, k, 20 + e % 4) for e in range(experts)]
    ye = [torch.empty((m, n), dtype=torch.bfloat16, device=dev) for _ in range(experts)]
    rec = np.zeros(experts, dtype=nv.GROUP_DTYPE)
    for e in range(experts):
        rec[e] = (xe[e].data_ptr(), ews[e][0].data_ptr(), ews[e][1].data_ptr(), ye[e].data_ptr(), t, m)
    table = torch.from_numpy(rec.view(np.uint8)).to(dev)
    us = timed_graph(torch, stream, lambda h: call(nv.linear_grouped_raw, table.data_ptr(), experts, m, n, k,
                                                   nv.OUT_BF16, h)) * 1e3
    fused[f"grouped_{experts}x{n}x{k}_M{m}"] = {"us": us, "weight_GBps": experts * wb / (us * 1e-6) / 1e9}
    del ews
    out["fused"] = fused

    fp8 = {}
    for s in workload.ROUND_SHAPES:
        codes, scales = nv.fp8_pack(workload.weights_f32(s.n, s.k, 21))
        c0, s0 = torch.from_numpy(codes).to(dev), torch.from_numpy(scales).to(dev)
        wb = codes.nbytes + scales.nbytes
        ws = rotate(lambda: (c0.clone(), s0.clone()), wb)
        for m in (1, 16, 32):
            x = xs(m, s.k, 22)
            y = torch.empty((m, s.n), dtype=torch.bfloat16, device=dev)
            def run(h):
                for c, sc in ws:
                    call(nv.fp8_linear_raw, x.data_ptr(), c.data_ptr(), sc.data_ptr(), y.data_ptr(), m, s.n, s.k,
                         nv.OUT_BF16, h)
            us = timed_graph(torch, stream, run) * 1e3 / len(ws)
            gbps = wb / (us * 1e-6) / 1e9
            fp8[f"{s.n}x{s.k}_M{m}"] = {"us": us, "weight_GBps": gbps, "frac_of_peak": gbps / PEAK_HBM_GBPS}
        # many rows: fp8_w8a16_gemm (what fp8_w8a16_matmul runs above 32 rows)
        for m in (64, 256, 1024):
            x = xs(m, s.k, 23)
            y = torch.empty((m, s.n), dtype=torch.bfloat16, device=dev)
            def run_g(h):
                for c, sc in ws:
                    call(nv.fp8_gemm_raw, x.data_ptr(), c.data_ptr(), sc.data_ptr(), y.data_ptr(), m, s.n, s.k,
                         nv.OUT_BF16, h)
            us = timed_graph(torch, stream, run_g) * 1e3 / len(ws)
            tf = 2.0 * m * s.n * s.k / (us * 1e-6) / 1e12
            fp8[f"gemm_{s.n}x{s.k}_M{m}"] = {"us": us, "weight_GBps": wb / (us * 1e-6) / 1e9, "TFLOPs": tf,
                                             "frac_of_bf16_mfma_peak": tf / PEAK_BF16_MFMA_TFLOPS}
        del ws
    out["fp8_w8a16"] = fp8
    torch.cuda.synchronize()
    return out


def cpu_baseline(torch, dev, rnd: Round, launches: dict, ms_list) -> dict:
    """The oracle on this host's cores over a bounded sample of the same
    workload: the decode round's products of its first layers, in round order
    at each timed M, until about CPU_BASELINE_MIN_S seconds of oracle time; each
    product's columns are split over one worker thread per core (NumPy's
    decode and matmul release the GIL), BLAS single-threaded per worker.  The
    GPU's outputs of the same products are checked against it."""
    import threadpoolctl
    import oracle
    cores = cpu_cores()
    total_s = 0.0
    weight_bytes = 0
    worst = 0.0
    done = []
    jobs = [(m, idx) for idx in range(4 * min(CPU_BASELINE_LAYERS, rnd.layers)) for m in ms_list]
    with threadpoolctl.threadpool_limits(limits=1, user_api="blas"), ThreadPoolExecutor(cores) as ex:
        for m, idx in jobs:
            if total_s >= CPU_BASELINE_MIN_S and len(done) >= len(ms_list) * 4:
                break
            if total_s >= CPU_BASELINE_MAX_S:
                break
            l, p, s, wp, sc, t = rnd.items[idx]
            lc = launches[m]
            xp, wpp, scp, tt, _, mm, n, k, _ = lc.calls[idx]
            y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
            st = lc.nv.linear_raw(xp, wpp, scp, tt, y.data_ptr(), mm, n, k, lc.nv.OUT_BF16,
                                  torch.cuda.current_stream().cuda_stream)
            assert st == lc.nv.OK
            torch.cuda.synchronize()
            packed, scales, t0 = rnd.host[(l, p)]
            xb = workload.activations_bf16(m, k, workload.round_act_seed(l, p, m))
            blocks = np.array_split(np.arange(n), cores)
            c0 = time.perf_counter()
            parts = list(ex.map(lambda cols: oracle.linear_ref(xb, packed, scales, t0, cols), blocks))
            total_s += time.perf_counter() - c0
            y_ref = np.concatenate(parts, axis=1)
            weight_bytes += packed.nbytes + scales.nbytes
            bnd = np.concatenate(list(ex.map(lambda cols: oracle.bound(xb, packed, scales, t0, cols), blocks)),
                                 axis=1)
            y64 = y.float().cpu().numpy().astype(np.float64)
            worst = max(worst, oracle.max_violation(y64, y_ref, bnd, "bf16"))
            done.append((l, p, m))
    return {"value": weight_bytes / total_s / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{len(done)} decode-round products in round order (layers {done[0][0]}..{done[-1][0]}, "
                      f"every projection, M = {', '.join(str(m) for m in ms_list)} each; last "
                      f"L{done[-1][0]} P{done[-1][1]} M{done[-1][2]}; {weight_bytes} weight-stream bytes) in "
                      f"{total_s:.1f} s of oracle time: fp64 decode and dgemm, columns split over {cores} "
                      f"worker threads, BLAS single-threaded per worker",
            "seconds": total_s, "parity_max_err_over_tol": worst}


def traffic_from_profile(kernel: str, m: int):
    """Calibrated HBM bytes per launch of `kernel` at `m` rows from the committed
    rocprofv3 counter summary, if it was taken on the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    for row in rec.get("kernels", []):
        if row.get("kernel") == kernel and row.get("m") == m:
            return row.get("hbm_bytes_per_launch")
    return None


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=workload.ROUND_LAYERS)
    ap.add_argument("--m", type=str, default="1,16,32", help="row counts timed in each step")
    ap.add_argument("--extra-m", type=str, default="8", help="row counts timed after the steps, reported only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the per-kernel, plain-read and other-workload timings")
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager launches instead of graph replays (for counter collection)")
    ap.add_argument("--copy-only", action="store_true",
                    help="only run a 1 GiB device copy 5 times (counter calibration) and exit")
    ap.add_argument("--next-only", action="store_true",
                    help="only time the other regimes and forms (GEMM, expand, fused, grouped, FP8) and exit")
    ap.add_argument("--warm-ms", type=float, default=WARM_MS,
                    help="replay each timed graph at least this long before timing it (0: two replays; "
                         "for counter collection, which does not need warm clocks)")
    args = ap.parse_args()
    globals()["WARM_MS"] = args.warm_ms

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the NVFP4 skinny product has no collective; "
              "run with --gpus 1", file=sys.stderr)
        return 2

    import torch
    import verify_nvfp4_w4a16_amd as nv

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_only:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read_per_dispatch": 1 << 30, "copy_bytes_written_per_dispatch": 1 << 30,
                          "dispatches": 5}), flush=True)
        return 0
    nv.init()
    if args.next_only:
        stream = torch.cuda.Stream(device=dev)
        print(json.dumps({"next": next_rows(torch, dev, stream),
                          "kernel_source_sha256_16": kernel_source_hash()}), flush=True)
        return 0
    ms_list = [int(v) for v in args.m.split(",") if v]
    extra_m = [int(v) for v in args.extra_m.split(",") if v]

    rnd = Round(torch, dev, args.layers)
    launches = {m: Launches(torch, dev, rnd, m) for m in ms_list + extra_m}
    stream = torch.cuda.Stream(device=dev)
    graphs = {}
    for m, lc in launches.items():
        lc.launch(torch.cuda.current_stream().cuda_stream)       # warm, eager
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            with torch.cuda.graph(g, stream=stream):
                lc.launch(stream.cuda_stream)
        torch.cuda.current_stream().wait_stream(stream)
        graphs[m] = g
    torch.cuda.synchronize()
    log(f"[bench] captured {len(graphs)} round graphs of {len(rnd.items)} launches")

    weight_bytes = rnd.weight_bytes()
    events = {m: [] for m in ms_list}
    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            for m in ms_list:
                graphs[m].replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            for m in ms_list:
                s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                s.record(stream)
                if args.no_graph:
                    launches[m].launch(stream.cuda_stream)
                else:
                    graphs[m].replay()
                e.record(stream)
                events[m].append((s, e))
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    log(f"[bench] timed {args.steps} steps in {wall:.3f}s")

    per_m = {}
    for m in ms_list:
        ms = [s.elapsed_time(e) for s, e in events[m]]
        med = float(np.median(ms))
        gbps = weight_bytes / (med * 1e-3) / 1e9
        per_m[str(m)] = {"round_ms_median": med, "round_ms_p10": float(np.percentile(ms, 10)),
                         "round_ms_p90": float(np.percentile(ms, 90)),
                         "weight_stream_GBps": gbps, "pct_of_peak": 100 * gbps / PEAK_HBM_GBPS,
                         "all_alg_bytes_GBps": rnd.algorithmic_bytes(m) / (med * 1e-3) / 1e9,
                         "us_per_launch": med * 1e3 / len(rnd.items)}
    for m in extra_m:
        ts = []
        with torch.cuda.stream(stream):
            for _ in range(max(3, args.steps)):
                s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                s.record(stream)
                graphs[m].replay()
                e.record(stream)
                ts.append((s, e))
        torch.cuda.synchronize()
        med = float(np.median([s.elapsed_time(e) for s, e in ts]))
        gbps = weight_bytes / (med * 1e-3) / 1e9
        per_m[str(m)] = {"round_ms_median": med, "weight_stream_GBps": gbps,
                         "pct_of_peak": 100 * gbps / PEAK_HBM_GBPS, "timed_in_steps": False}
    for g in graphs.values():
        del g
    graphs.clear()

    kernels, ceiling, configs = None, None, None
    roofline = None
    if not args.no_extras:
        kernels = per_kernel(torch, stream, rnd, launches, ms_list)
        dom = max(kernels, key=lambda r: r["round_share_us"])
        achieved = dom["weight_GBps"]
        roofline = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                    "frac": achieved / PEAK_HBM_GBPS,
                    "traffic": traffic_from_profile(dom["kernel"], dom["m"]),
                    "kernel": dom["kernel"], "m": dom["m"], "shapes": dom["shapes"],
                    "launches_per_round": dom["launches_per_round"],
                    "avg_launch_us": dom["avg_launch_us"],
                    "alg_bytes_per_launch": dom["weight_bytes_per_launch"],
                    "alg_bytes_rule": "0.5625 B per weight (packed e2m1 + e4m3 scale) x N x K, "
                                      "averaged over the kernel's launches",
                    "xy_bytes_per_launch": dom["xy_bytes_per_launch"],
                    "mfma_frac_of_bf16_peak": dom["mfma_TFLOPs"] / PEAK_BF16_MFMA_TFLOPS}
        ceiling = read_ceiling(torch, stream, rnd)
        configs = config_timings(torch, dev, stream)
        configs["next"] = next_rows(torch, dev, stream)

    base = None
    if not args.no_cpu_baseline:
        base = cpu_baseline(torch, dev, rnd, launches, ms_list)

    total_bytes = weight_bytes * len(ms_list) * args.steps
    value = total_bytes / wall / 1e9
    out = {
        "metric": "weight-stream HBM GB/s (% of peak) for NVFP4 skinny GEMM at M=1,16,32",
        "launch": "eager" if args.no_graph else "hip-graph",
        "value": value, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"decode round: {args.layers} layers x {{(8192,4096), (4096,8192), "
                               "(24576,4096), (4096,12288)} NVFP4 W4A16, back-to-back per M, HIP graph",
                   "m": ms_list, "layers": args.layers, "launches_per_round": len(rnd.items),
                   "weight_stream_bytes_per_round": weight_bytes, "parallelism": "single GPU"},
        "pct_of_peak": 100 * value / PEAK_HBM_GBPS,
        "per_m": per_m,
        "roofline": roofline,
        "cpu_baseline": base,
        "plain_read_ceiling": ceiling,
        "kernels": kernels,
        "configs": configs,
        "copy_GBps_read_plus_write": copy_bandwidth(torch, dev),
        "kernel_source_sha256_16": kernel_source_hash(),
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
