"""Decode-round benchmark of the NVFP4 W4A16 skinny product on one MI355X.

Workload: 48 layers x {(8192,4096), (4096,8192), (24576,4096), (4096,12288)}
NVFP4 weights (10,468,982,784 weights; 5,888,802,816 bytes of packed nibbles
plus e4m3 scales), weights N(0, 0.02) packed by nvfp4_pack, bf16 N(0,1)
activations drawn per (layer, projection, M).  One step runs the whole round
back-to-back on one stream at each M in {1, 16, 32}, each round replayed from
one captured HIP graph of 192 nvfp4_linear launches.

value: weight-stream GB/s = packed + scale bytes of every timed product over
the timed wall time (decimal GB/s), all three M together; per-M figures and %
of the 8.0 TB/s MI355X peak are in "per_m".  Prints one JSON line on stdout.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workload  # noqa: E402

PEAK_HBM_GBPS = 8000.0
CPU_BASELINE_LAYERS = 2   # layers whose products the oracle times (about 10 s of CPU work)
KERNEL_SOURCE = os.path.join(ROOT, "verify_nvfp4_w4a16_amd", "csrc", "kernels", "nvfp4_linear.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_decode_round.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_budget() -> int:
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:
        return max(1, min(16, os.cpu_count() or 1))


def kernel_source_hash() -> str:
    """SHA-256 prefix of the kernel source with its comment lines and blank
    lines removed, so a counter profile stays attached to the code it
    measured across comment-only edits."""
    with open(KERNEL_SOURCE, encoding="utf-8") as f:
        code = [ln.rstrip() for ln in f if ln.strip() and not ln.lstrip().startswith("//")]
    return hashlib.sha256("\n".join(code).encode()).hexdigest()[:16]


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
        with ThreadPoolExecutor(max(1, cpu_budget() // 2)) as ex:
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
    """Activations and outputs of one round at row count m, launched on `stream`."""

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

    def launch_all(self, stream_handle: int) -> None:
        nv = self.nv
        for xp, wpp, scp, t, yp, m, n, k, _ in self.calls:
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


def cpu_baseline(torch, dev, rnd: Round, graphs: dict, launches: dict, ms_list) -> dict:
    """The oracle on this host's cores over a bounded sample (the four
    products of the first CPU_BASELINE_LAYERS layers at each timed M, about
    10 s), checked against the GPU's output for the same products; reported,
    never optimised."""
    import threadpoolctl
    import oracle
    total_s = 0.0
    weight_bytes = 0
    worst = 0.0
    for m in ms_list:
        # GPU outputs of those products: rerun their launches eagerly
        lc = launches[m]
        for idx, (l, p, s, wp, sc, t) in enumerate(rnd.items[:4 * CPU_BASELINE_LAYERS]):
            xp, wpp, scp, tt, yp, mm, n, k, x = lc.calls[idx]
            y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
            st = lc.nv.linear_raw(xp, wpp, scp, tt, y.data_ptr(), mm, n, k, lc.nv.OUT_BF16,
                                  torch.cuda.current_stream().cuda_stream)
            assert st == lc.nv.OK
            torch.cuda.synchronize()
            packed, scales, t0 = rnd.host[(l, p)]
            xb = workload.activations_bf16(m, k, workload.round_act_seed(l, p, m))
            c0 = time.perf_counter()
            y_ref = oracle.linear_ref(xb, packed, scales, t0)
            total_s += time.perf_counter() - c0
            weight_bytes += packed.nbytes + scales.nbytes
            bnd = oracle.bound(xb, packed, scales, t0)
            y64 = y.float().cpu().numpy().astype(np.float64)
            worst = max(worst, oracle.max_violation(y64, y_ref, bnd, "bf16"))
    blas = [i for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas"]
    threads = max([i["num_threads"] for i in blas] or [1])
    return {"value": weight_bytes / total_s / 1e9, "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"the 4 products of layers 0..{CPU_BASELINE_LAYERS - 1} at M={','.join(map(str, ms_list))} "
                      f"({weight_bytes} weight-stream bytes, {total_s:.1f} s; fp64 decode "
                      f"single-threaded, BLAS dgemm on {threads} threads)",
            "seconds": total_s, "parity_max_err_over_tol": worst}


def kernel_name(m: int) -> str:
    """The kernel nvfp4_linear runs for the decode round's products at M rows
    (the dispatch rule of the library: per-tile kernel up to 4 rows, else the
    many-row kernel for these shapes, whose x does not fit one LDS)."""
    if m <= 4:
        return f"nvfp4_skinny_tile<1, 1, NB, bf16> (per-tile kernel, M={m} round)"
    if m <= 16:
        return (f"nvfp4_skinny_split<1, 1, W, bf16> (many-row kernel, M={m} round; "
                f"W = 6 for the 24576-column product, 4 for the others)")
    return (f"nvfp4_skinny_split<1, 2, W, bf16> (many-row kernel, M={m} round; "
            f"W = 6 for the 24576-column product, 8 for the others)")


def traffic_from_profile(per_launch_alg: float):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=workload.ROUND_LAYERS)
    ap.add_argument("--m", type=str, default="1,16,32", help="row counts timed in each step")
    ap.add_argument("--extra-m", type=str, default="8", help="row counts timed after the steps, reported only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true", help="also time eager launches")
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager launches instead of graph replays (for counter collection)")
    ap.add_argument("--copy-only", action="store_true",
                    help="only run a 1 GiB device copy 5 times (counter calibration) and exit")
    args = ap.parse_args()

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
    ms_list = [int(v) for v in args.m.split(",") if v]
    extra_m = [int(v) for v in args.extra_m.split(",") if v]

    rnd = Round(torch, dev, args.layers)
    launches = {m: Launches(torch, dev, rnd, m) for m in ms_list + extra_m}
    stream = torch.cuda.Stream(device=dev)
    graphs = {}
    for m, lc in launches.items():
        lc.launch_all(torch.cuda.current_stream().cuda_stream)       # warm, eager
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            with torch.cuda.graph(g, stream=stream):
                lc.launch_all(stream.cuda_stream)
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
                    launches[m].launch_all(stream.cuda_stream)
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

    eager = None
    if args.eager:
        eager = {}
        for m in ms_list:
            torch.cuda.synchronize()
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            for _ in range(3):
                launches[m].launch_all(torch.cuda.current_stream().cuda_stream)
            e.record()
            e.synchronize()
            eager[str(m)] = weight_bytes / (s.elapsed_time(e) / 3 * 1e-3) / 1e9

    # Roofline of the dominant kernel: the row count whose round takes longest.
    dom = max(ms_list, key=lambda m: per_m[str(m)]["round_ms_median"])
    launches_per_round = len(rnd.items)
    avg_launch_s = per_m[str(dom)]["round_ms_median"] * 1e-3 / launches_per_round
    alg_per_launch = rnd.algorithmic_bytes(dom) / launches_per_round
    achieved = alg_per_launch / avg_launch_s / 1e9
    traffic = traffic_from_profile(alg_per_launch)
    roofline = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBPS, "traffic": traffic,
                "kernel": kernel_name(dom),
                "alg_bytes_per_launch": alg_per_launch, "avg_launch_us": avg_launch_s * 1e6}

    base = None
    if not args.no_cpu_baseline:
        base = cpu_baseline(torch, dev, rnd, graphs, launches, ms_list)

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
                   "m": ms_list, "layers": args.layers, "launches_per_round": launches_per_round,
                   "weight_stream_bytes_per_round": weight_bytes, "parallelism": "single GPU"},
        "pct_of_peak": 100 * value / PEAK_HBM_GBPS,
        "per_m": per_m,
        "roofline": roofline,
        "cpu_baseline": base,
        "copy_GBps_read_plus_write": copy_bandwidth(torch, dev),
        "kernel_source_sha256_16": kernel_source_hash(),
    }
    if eager is not None:
        out["eager_weight_stream_GBps"] = eager
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
