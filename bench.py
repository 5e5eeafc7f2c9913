#!/usr/bin/env python3
"""SGEMM benchmark on one MI355X: GFLOPS at M=N=K=4096 (C = alpha*A*B + beta*C,
row-major FP32, alpha=1, beta=0), as a fraction of measured and published
FP32 peaks.

Default run (the contract): ``python bench.py [--gpus 1] [--steps K] [--warmup W]``
prints ONE JSON line.  A "step" is one sgemm() call on the 4096^3 problem, with
A, B and C already resident in device memory.  After W untimed steps (and a
clock-waking burst, see ``wake``), exactly K steps are timed between two device
synchronisations; each launch is also bracketed by HIP events on the stream it
is launched on, which gives the average kernel duration for the roofline.

Other modes (one JSON line per result, not the contract line):
  --sweep            every square size and rectangular shape, auto choice
  --variants         every kernel variant on the 4096^3 problem
  --shape M N K      a single shape (with --variant V to force a variant)
  --profile          only the timed steps, no ceilings or CPU baseline: the
                     command to run under rocprofv3

Accounting (as on the pages): FLOPs = 2*M*N*K, the epilogue is not counted
("Optimizing SGEMM in CUDA" and "The road to a fast GEMM", section "The
problem and the ceiling"); algorithmic bytes = 4*(M*K + K*N + M*N), plus
4*M*N when beta != 0 (C read and written).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X published figures (AMD datasheet): dense FP32 matrix and vector
# 157.3 TFLOP/s, HBM3E 8 TB/s; 256 CUs.
PEAK_FP32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
NUM_CUS = 256

METRIC = "SGEMM GFLOPS at M=N=K=4096 on 1 MI355X; % of measured FP32 peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_sgemm_4096.json")


def flops(M: int, N: int, K: int) -> float:
    """Floating-point operations of one GEMM: 2*M*N*K."""
    return 2.0 * M * N * K


def min_bytes(M: int, N: int, K: int, beta: float = 0.0) -> float:
    """Bytes a GEMM must move at least: read A and B, write C, and read C
    too when beta != 0."""
    b = 4.0 * (M * K + K * N + M * N)
    if beta != 0.0:
        b += 4.0 * M * N
    return b


def arithmetic_intensity(M, N, K, beta=0.0) -> float:
    return flops(M, N, K) / min_bytes(M, N, K, beta)


def tile_global_bytes(M: int, N: int, K: int, BM: int, BN: int) -> float:
    """Bytes a tiled kernel loads from global memory (L2 or HBM) for A and B:
    each of the ceil(M/BM)*ceil(N/BN) tiles reads BM rows of A and BN columns
    of B over the whole of K ("The road to a fast GEMM", Exercise 1)."""
    tiles = -(-M // BM) * -(-N // BN)
    return tiles * 4.0 * (BM + BN) * K


def lds_reads_per_fma(TM: int, TN: int) -> float:
    """Operand reads per multiply-add for a TM x TN register tile: an outer
    product of TM values of A and TN of B feeds TM*TN multiply-adds."""
    return (TM + TN) / float(TM * TN)


# The sources that define the matrix-core kernel whose counters are stored.
KERNEL_FILES = ("sgemm_sched.hpp", "sgemm_mfma_sched.hip", "sgemm_mfma.hpp", "sgemm_mfma.hip",
                "sgemm_tiles.hpp", "sgemm_common.hpp")


def kernel_source_hash(files=KERNEL_FILES) -> str:
    """Hash of the kernel's HIP sources, so stored counter readings can be
    matched to the code they were taken from."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "dense_fp32_gemm_sgemm_amd", "csrc")
    for name in sorted(files):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


# Names of the matrix-core GEMM kernels as the profiler prints them.
GEMM_KERNEL_PREFIXES = ("void sg950::mfma_kernel", "void sg950::sched_kernel")


def _counter_means(path, kernel_prefix):
    """Mean counter value per counter name over the dispatches of kernels whose
    name starts with kernel_prefix (a string or a tuple of strings), from a
    rocprofv3 counter_collection.csv."""
    import csv
    vals = {}
    names = set()
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Kernel_Name"].startswith(kernel_prefix):
                vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
                names.add(r["Kernel_Name"])
    return {k: sum(v) / len(v) for k, v in vals.items()}, sorted(names), {k: len(v) for k, v in vals.items()}


def traffic_from_counters(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, variant,
                          copy_bytes=256 * 1024 * 1024):
    """HBM-side bytes per launch of the GEMM kernel from FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch), each scaled by what the same counter reads
    for a streaming copy that reads and writes copy_bytes."""
    gemm_prefix = GEMM_KERNEL_PREFIXES
    f, fnames, fn = _counter_means(fetch_csv, gemm_prefix)
    w, _, wn = _counter_means(write_csv, gemm_prefix)
    cf, _, _ = _counter_means(copy_fetch_csv, "sg950::copy_kernel")
    cw, _, _ = _counter_means(copy_write_csv, "sg950::copy_kernel")
    fetch_scale = copy_bytes / (cf["FETCH_SIZE"] * 1024.0)
    write_scale = copy_bytes / (cw["WRITE_SIZE"] * 1024.0)
    fetch_b = f["FETCH_SIZE"] * 1024.0 * fetch_scale
    write_b = w["WRITE_SIZE"] * 1024.0 * write_scale
    return {"variant": variant, "kernel": fnames, "source_hash": kernel_source_hash(),
            "fetch_kib_raw": f["FETCH_SIZE"], "write_kib_raw": w["WRITE_SIZE"],
            "dispatches": {"fetch": fn["FETCH_SIZE"], "write": wn["WRITE_SIZE"]},
            "copy_fetch_kib_raw": cf["FETCH_SIZE"], "copy_write_kib_raw": cw["WRITE_SIZE"],
            "fetch_scale": fetch_scale, "write_scale": write_scale,
            "fetch_bytes_per_launch": fetch_b, "write_bytes_per_launch": write_b,
            "bytes_per_launch": fetch_b + write_b,
            "algorithmic_bytes_per_launch": min_bytes(4096, 4096, 4096, 0.0)}


# ---------------------------------------------------------------- GPU side

def _torch():
    import torch
    return torch


def wake(seconds: float, fn):
    """Run `fn` back to back for about `seconds` so the clocks are up before
    timing (the Tinyforge README's benchmark-hygiene note: short kernels after
    host work run at idle clocks)."""
    torch = _torch()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()


def time_steps(fn, steps: int, stream):
    """Times `steps` calls of fn: returns (total ms from the first event to the
    last, list of per-launch ms from events around each launch)."""
    torch = _torch()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        starts[i].record(stream)
        fn()
        ends[i].record(stream)
    torch.cuda.synchronize()
    per = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    total = starts[0].elapsed_time(ends[-1])
    return total, per


class Problem:
    """Device buffers of one GEMM and a zero-overhead launcher."""

    def __init__(self, M, N, K, alpha=1.0, beta=0.0, seed=0, kind="real", ops="NN", batch=1):
        torch = _torch()
        import numpy as np
        from workloads import draw
        self.M, self.N, self.K, self.alpha, self.beta = M, N, K, alpha, beta
        self.ta, self.tb = ops[0] == "T", ops[1] == "T"
        self.batch = batch
        A, B, C = draw(M, N, K, seed=seed, kind=kind, with_c=(beta != 0.0))
        self.host = (A, B, C)
        # stored matrices: the transposes when the operation transposes them
        As = np.ascontiguousarray(A.T) if self.ta else A
        Bs = np.ascontiguousarray(B.T) if self.tb else B
        self.lda, self.ldb = max(1, As.shape[1]), max(1, Bs.shape[1])
        # a batch repeats the drawn slice (the timing does not depend on values)
        self.A = torch.from_numpy(As).cuda().repeat(batch, 1, 1) if batch > 1 else torch.from_numpy(As).cuda()
        self.B = torch.from_numpy(Bs).cuda().repeat(batch, 1, 1) if batch > 1 else torch.from_numpy(Bs).cuda()
        Cd = (torch.from_numpy(C).cuda() if C is not None
              else torch.zeros((M, N), dtype=torch.float32, device="cuda"))
        self.C = Cd.repeat(batch, 1, 1) if batch > 1 else Cd
        self.strides = ((self.A.stride(0), self.B.stride(0), self.C.stride(0)) if batch > 1
                        else (0, 0, 0))
        self.stream = torch.cuda.current_stream()

    def launcher(self, variant=-1):
        import dense_fp32_gemm_sgemm_amd as sg
        sa, sb, sc = self.strides
        args = (int(self.ta), int(self.tb), self.M, self.N, self.K, float(self.alpha),
                self.A.data_ptr(), self.lda, sa, self.B.data_ptr(), self.ldb, sb, float(self.beta),
                self.C.data_ptr(), max(1, self.N), sc, self.batch, self.stream.cuda_stream, variant)
        fn_ex = sg.load().sgemm_strided_batched_ex

        def fn():
            st = fn_ex(*args)
            if st != 0:
                raise RuntimeError("sgemm status %d: %s" % (st, sg.sgemm_status_string(st)))
        return fn

    def variant_name(self, variant=-1):
        import dense_fp32_gemm_sgemm_amd as sg
        if variant >= 0:
            return sg.sgemm_variant_name(variant)
        sa, sb, sc = self.strides
        v = sg.sgemm_strided_batched_select_variant(
            int(self.ta), int(self.tb), self.M, self.N, self.K, self.alpha, self.A.data_ptr(),
            self.lda, sa, self.B.data_ptr(), self.ldb, sb, self.beta, self.C.data_ptr(),
            max(1, self.N), sc, self.batch)
        return sg.sgemm_variant_name(v) if v >= 0 else "none"


def measure_ceilings(samples: int = 15):
    """Measured FP32 matrix-core, FP32 vector and HBM copy rates."""
    torch = _torch()
    import dense_fp32_gemm_sgemm_amd as sg
    stream = torch.cuda.current_stream()
    h = stream.cuda_stream
    blocks = NUM_CUS * 8
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    out = {}

    def rate(launch, target_ms=20.0):
        # calibrate the iteration count to about target_ms per launch
        iters = 256
        while True:
            st, fl = launch(iters)
            assert st == 0
            torch.cuda.synchronize()
            t0 = torch.cuda.Event(enable_timing=True)
            t1 = torch.cuda.Event(enable_timing=True)
            t0.record(stream)
            launch(iters)
            t1.record(stream)
            torch.cuda.synchronize()
            ms = t0.elapsed_time(t1)
            if ms >= target_ms * 0.5 or iters >= 1 << 22:
                break
            iters = int(iters * max(2.0, target_ms / max(ms, 1e-3)))
        wake(0.5, lambda: launch(iters))
        vals = []
        for _ in range(samples):
            t0 = torch.cuda.Event(enable_timing=True)
            t1 = torch.cuda.Event(enable_timing=True)
            t0.record(stream)
            _, fl = launch(iters)
            t1.record(stream)
            torch.cuda.synchronize()
            vals.append(fl / (t0.elapsed_time(t1) * 1e-3) / 1e12)
        return statistics.median(vals), vals

    out["mfma_f32_32x32x2_tflops"], _ = rate(lambda it: sg.sgemm_ceiling_mfma(32, blocks, it, sink.data_ptr(), h))
    out["mfma_f32_16x16x4_tflops"], _ = rate(lambda it: sg.sgemm_ceiling_mfma(16, blocks, it, sink.data_ptr(), h))
    out["valu_fma_f32_tflops"], _ = rate(lambda it: sg.sgemm_ceiling_fma(blocks, it, sink.data_ptr(), h))
    n = 256 * 1024 * 1024  # 1 GiB per buffer
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty(n, dtype=torch.float32, device="cuda")
    cp = lambda: sg.sgemm_ceiling_copy(src.data_ptr(), dst.data_ptr(), n, NUM_CUS * 16, h)
    wake(0.2, cp)
    vals = []
    for _ in range(samples):
        total, _ = time_steps(cp, 1, stream)
        vals.append(2 * 4 * n / (total * 1e-3) / 1e9)
    out["hbm_copy_gbs"] = statistics.median(vals)
    del src, dst
    return out


def clock_under_load(fn, settle_s: float = 1.0, limit_s: float = 20.0):
    """GPU clocks while `fn` (one launch) runs back to back: `amd-smi metric
    -c` is started after `settle_s` seconds of load and the launches go on
    until it has answered.  Returns the gfx clocks (MHz) of the busiest GPU it
    lists, or None when the tool is missing or fails (best effort only)."""
    import shutil
    import subprocess
    exe = shutil.which("amd-smi") or "/opt/rocm/bin/amd-smi"
    if not os.path.exists(exe):
        return None
    torch = _torch()
    proc = None
    t0 = time.time()
    try:
        while time.time() - t0 < limit_s:
            for _ in range(10):
                fn()
            torch.cuda.synchronize()
            if proc is None and time.time() - t0 > settle_s:
                proc = subprocess.Popen([exe, "metric", "-c", "--json"], stdout=subprocess.PIPE,
                                        stderr=subprocess.DEVNULL)
            if proc is not None and proc.poll() is not None:
                break
        if proc is None:
            return None
        if proc.poll() is None:
            proc.kill()
            proc.wait()
            return None
        data = json.loads(proc.stdout.read())
        best = None
        for gpu in data.get("gpu_data", []):
            clk = gpu.get("clock", {})
            gfx = [v["clk"]["value"] for k, v in clk.items() if k.startswith("gfx_")
                   and isinstance(v.get("clk", {}).get("value"), (int, float))]
            top = [v["max_clk"]["value"] for k, v in clk.items() if k.startswith("gfx_")
                   and isinstance(v.get("max_clk", {}).get("value"), (int, float))]
            if gfx and (best is None or statistics.mean(gfx) > best["gfx_mhz_mean"]):
                best = {"gfx_mhz_mean": round(statistics.mean(gfx), 1), "gfx_mhz_min": min(gfx),
                        "gfx_mhz_max": max(gfx), "gfx_mhz_limit": max(top) if top else None,
                        "source": "amd-smi metric -c during back-to-back launches of the timed kernel"}
        return best
    except Exception:
        if proc is not None and proc.poll() is None:
            proc.kill()
            proc.wait()
        return None


def cpu_baseline(target_s: float = 12.0):
    """The oracle (as it stands) on a bounded row sample of the 4096^3
    workload, on the host cores."""
    import numpy as np
    import oracle
    from workloads import HEADLINE, draw_workload, sweep_workloads
    A, B, _ = draw_workload(HEADLINE)
    squares = {w.M: w for w in sweep_workloads()}
    oracle.load()
    rows = 32
    t0 = time.perf_counter()
    oracle.gemm(A, B, rows=np.arange(rows))
    dt = time.perf_counter() - t0
    nrows = int(min(HEADLINE.M, max(rows, rows * target_s / max(dt, 1e-6))))
    sel = np.arange(nrows)
    t0 = time.perf_counter()
    oracle.gemm(A, B, rows=sel)
    dt = time.perf_counter() - t0
    gfl = flops(nrows, HEADLINE.N, HEADLINE.K) / dt / 1e9
    # The other sizes the oracle is quoted at: all of 256^3, and a row sample
    # of 8192^3 (about a second of CPU time together).
    by_size = {}
    for n, r in ((256, 256), (8192, 128)):
        An, Bn, _ = draw_workload(squares[n])
        t0 = time.perf_counter()
        oracle.gemm(An, Bn, rows=np.arange(r))
        by_size["%d^3 (%d rows)" % (n, r)] = round(flops(r, n, n) / (time.perf_counter() - t0) / 1e9, 3)
        del An, Bn
    return {"value": round(gfl, 3), "unit": "GFLOPS", "cores": oracle.max_threads(),
            "kind": "oracle",
            "sample": "first %d of 4096 output rows of the 4096^3 workload (fp64 i-k-j "
                      "oracle, OpenMP over rows), %.1f s" % (nrows, dt),
            "by_size": by_size}


def stored_traffic(variant: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel sources and the same variant."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != kernel_source_hash() or t.get("variant") != variant:
        return None
    return round(t.get("bytes_per_launch"))


def vendor_context(prob: Problem, steps: int, warmup: int):
    """torch.mm on the same device tensors with TF32 off: the vendor BLAS in
    strict FP32, timed the same way.  A reported stopwatch, not part of the
    library; beta = 0 problems only (torch.mm overwrites its output)."""
    torch = _torch()
    if prob.beta != 0.0 or prob.ta or prob.tb:
        return {}
    prev = torch.backends.cuda.matmul.allow_tf32
    torch.backends.cuda.matmul.allow_tf32 = False
    try:
        A, B, C = prob.A, prob.B, prob.C
        fn = lambda: torch.mm(A, B, out=C)
        for _ in range(warmup):
            fn()
        wake(0.25, fn)
        _, per = time_steps(fn, steps, torch.cuda.current_stream())
    finally:
        torch.backends.cuda.matmul.allow_tf32 = prev
    ms = statistics.median(per)
    return {"torch_mm_fp32_ms_median": round(ms, 5),
            "torch_mm_fp32_gflops": round(flops(prob.M, prob.N, prob.K) / (ms * 1e-3) / 1e9, 1)}


def bench_problem(prob: Problem, steps: int, warmup: int, variant=-1):
    fn = prob.launcher(variant)
    for _ in range(warmup):
        fn()
    wake(0.25, fn)
    total, per = time_steps(fn, steps, prob.stream)
    return total, per


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=int(os.environ.get("WORLD_SIZE", "1")))
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--variant", type=int, default=-1)
    ap.add_argument("--shape", type=int, nargs=3, metavar=("M", "N", "K"))
    ap.add_argument("--beta", type=float, default=0.0)
    ap.add_argument("--batch", type=int, default=1,
                    help="strided batch of this many slices (non-contract modes)")
    ap.add_argument("--ops", default="NN", choices=["NN", "NT", "TN", "TT"],
                    help="op(A) op(B) for the non-contract modes (T = transposed operand)")
    ap.add_argument("--alpha", type=float, default=1.0)
    ap.add_argument("--sweep", action="store_true")
    ap.add_argument("--variants", action="store_true")
    ap.add_argument("--profile", action="store_true")
    ap.add_argument("--matrix", action="store_true",
                    help="every variant on every sweep and rectangular shape")
    ap.add_argument("--traffic-from", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="write the stored traffic figure from four counter_collection.csv files")
    ap.add_argument("--copy-calib", action="store_true",
                    help="one 256 MiB streaming copy (to scale HBM byte counters)")
    ap.add_argument("--few-rows", action="store_true",
                    help="few-rows grid (M <= 32, both orientations of B): the automatic choice, "
                         "the three candidate kernels and the vendor BLAS")
    ap.add_argument("--vendor", action="store_true",
                    help="with --sweep/--shape: also time torch.mm in strict FP32 (context only)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true")
    args = ap.parse_args(argv)

    if args.traffic_from:
        from_ = args.traffic_from
        # the variant the automatic choice runs on the 4096^3 problem (no GPU needed)
        import dense_fp32_gemm_sgemm_amd as sg
        v = sg.sgemm_select_variant(4096, 4096, 4096, 1.0, 256, 4096, 256, 4096, 0.0, 256, 4096)
        t = traffic_from_counters(*from_, variant=sg.sgemm_variant_name(v))
        os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(t, f, indent=1)
        print(json.dumps(t))
        return 0

    if args.gpus != 1:
        print("bench.py measures one GPU: this SGEMM runs whole on a single MI355X and "
              "--gpus %d is not supported (the sharded design is described, not built)"
              % args.gpus, file=sys.stderr)
        return 2

    torch = _torch()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    import dense_fp32_gemm_sgemm_amd as sg
    sg.load()

    if args.few_rows:
        return few_rows(args)
    if args.sweep or args.variants or args.shape or args.profile or args.matrix or args.copy_calib:
        return run_modes(args)

    M = N = K = 4096
    prob = Problem(M, N, K, 1.0, 0.0, seed=0)
    vname = prob.variant_name(args.variant)
    total, per = bench_problem(prob, args.steps, args.warmup, args.variant)
    ms_step = total / args.steps
    kern_ms = statistics.mean(per)
    value = flops(M, N, K) / (ms_step * 1e-3) / 1e9
    achieved = flops(M, N, K) / (kern_ms * 1e-3) / 1e12

    clocks = None if args.no_ceilings else clock_under_load(prob.launcher(args.variant))
    ceilings = None if args.no_ceilings else measure_ceilings()
    cpu = None if args.no_cpu_baseline else cpu_baseline()
    traffic = stored_traffic(vname)

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "sgemm M=N=K=4096 alpha=1 beta=0 row-major fp32, A,B uniform[-1,1] seed 0",
                   "M": M, "N": N, "K": K, "alpha": 1.0, "beta": 0.0, "variant": vname,
                   "parallelism": "single-gpu"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_FP32_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP32_TFLOPS, 4),
                     "traffic": traffic,
                     "kernel_ms_mean": round(kern_ms, 5),
                     "kernel_ms_median": round(statistics.median(per), 5),
                     "kernel_ms_std": round(statistics.pstdev(per), 5),
                     "kernel_ms_min": round(min(per), 5), "kernel_ms_max": round(max(per), 5)},
        "cpu_baseline": cpu,
        "gpu_clocks": clocks,
    }
    if ceilings:
        mf = ceilings["mfma_f32_32x32x2_tflops"]
        line["measured_ceilings"] = {k: round(v, 2) for k, v in ceilings.items()}
        line["pct_of_measured_mfma_f32"] = round(100.0 * value / 1e3 / mf, 2)
        line["pct_of_measured_valu_f32"] = round(100.0 * value / 1e3 / ceilings["valu_fma_f32_tflops"], 2)
        line["pct_of_datasheet_fp32"] = round(100.0 * value / 1e3 / PEAK_FP32_TFLOPS, 2)
    print(json.dumps(line), flush=True)
    return 0


FEW_ROWS_M = (1, 4, 8, 12, 16, 20, 24, 32)
FEW_ROWS_NK = ((4096, 4096), (8192, 8192), (16384, 16384), (1024, 4096), (2048, 2048),
               (4096, 1024), (4096, 16384), (65536, 1024))


def few_rows(args):
    """Median kernel time (us) of the automatic choice, of each few-rows
    candidate forced (vector-unit kernel, split-K 64x64 tiles, matrix-core
    kernel) and of torch.mm in strict FP32, per shape and orientation of B."""
    import dense_fp32_gemm_sgemm_amd as sg
    torch = _torch()
    names = sg.variant_names()
    cands = [names.index(n) for n in ("skinny_m8", "mfma16_64x64x64_4x2_pipe_splitk", "fewrows_m32")]
    for M in FEW_ROWS_M:
        for N, K in FEW_ROWS_NK:
            for ops in ("NN", "NT"):
                prob = Problem(M, N, K, ops=ops)
                rec = {"mode": "few-rows", "M": M, "N": N, "K": K, "ops": ops,
                       "auto": prob.variant_name(-1)}
                for v in [-1] + cands:
                    _, per = bench_problem(prob, args.steps, min(args.warmup, args.steps), v)
                    rec["us_" + ("auto" if v < 0 else names[v])] = round(statistics.median(per) * 1e3, 2)
                prev = torch.backends.cuda.matmul.allow_tf32
                torch.backends.cuda.matmul.allow_tf32 = False
                try:
                    Bm = prob.B.t() if prob.tb else prob.B
                    fn = lambda: torch.mm(prob.A, Bm, out=prob.C)
                    for _ in range(min(args.warmup, args.steps)):
                        fn()
                    wake(0.1, fn)
                    _, per = time_steps(fn, args.steps, torch.cuda.current_stream())
                finally:
                    torch.backends.cuda.matmul.allow_tf32 = prev
                rec["us_torch_mm_fp32"] = round(statistics.median(per) * 1e3, 2)
                print(json.dumps(rec), flush=True)
                del prob
                torch.cuda.empty_cache()
    return 0


def run_modes(args):
    from workloads import RAGGED_SHAPES, SHARD_SHAPES, SWEEP_SIZES
    import dense_fp32_gemm_sgemm_amd as sg
    jobs = []
    if args.copy_calib:
        torch = _torch()
        n = 64 * 1024 * 1024  # 256 MiB per buffer
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty(n, dtype=torch.float32, device="cuda")
        h = torch.cuda.current_stream().cuda_stream
        for _ in range(3):
            assert sg.sgemm_ceiling_copy(src.data_ptr(), dst.data_ptr(), n, NUM_CUS * 16, h) == 0
        torch.cuda.synchronize()
        print(json.dumps({"mode": "copy-calib", "bytes_read": 4 * n, "bytes_written": 4 * n,
                          "dispatches": 3}), flush=True)
        return 0
    if args.profile:
        shape = tuple(args.shape) if args.shape else (4096, 4096, 4096)
        prob = Problem(*shape, args.alpha, args.beta, seed=0, ops=args.ops)
        total, per = bench_problem(prob, args.steps, args.warmup, args.variant)
        kern_ms = statistics.mean(per)
        print(json.dumps({"mode": "profile", "shape": shape, "variant": prob.variant_name(args.variant),
                          "steps": args.steps, "kernel_ms_mean": round(kern_ms, 5),
                          "tflops": round(flops(*shape) / (kern_ms * 1e-3) / 1e12, 2)}), flush=True)
        return 0
    if args.sweep:
        jobs = ([((n, n, n), -1) for n in SWEEP_SIZES] + [(s, -1) for s in RAGGED_SHAPES] +
                [(s, -1) for s in SHARD_SHAPES])
    elif args.matrix:
        shapes = [(n, n, n) for n in SWEEP_SIZES] + list(RAGGED_SHAPES) + list(SHARD_SHAPES)
        jobs = [(sh, v) for sh in shapes for v in range(sg.sgemm_num_variants())
                if not (sg.sgemm_variant_name(v) == "simple" and flops(*sh) > 2e10)]
    elif args.variants:
        shape = tuple(args.shape) if args.shape else (4096, 4096, 4096)
        jobs = [(shape, v) for v in range(sg.sgemm_num_variants())]
    elif args.shape:
        jobs = [(tuple(args.shape), args.variant)]
    for shape, v in jobs:
        M, N, K = shape
        prob = Problem(M, N, K, args.alpha, args.beta, seed=0, ops=args.ops, batch=args.batch)
        name = prob.variant_name(v)
        work = flops(M, N, K) * args.batch
        steps = max(5, min(args.steps, int(2e12 / max(work, 1.0))))
        if name == "simple" and work > 1e11:
            steps = 3
        total, per = bench_problem(prob, steps, min(args.warmup, steps), v)
        kern_ms = statistics.median(per)
        rec = {"mode": "sweep" if args.sweep else ("matrix" if args.matrix else "variant"),
               "ops": args.ops, "batch": args.batch, "M": M, "N": N, "K": K,
               "beta": args.beta, "variant": name, "steps": steps,
               "kernel_ms_median": round(kern_ms, 5), "kernel_ms_min": round(min(per), 5),
               "gflops": round(work / (kern_ms * 1e-3) / 1e9, 1),
               "frac_fp32_peak": round(work / (kern_ms * 1e-3) / 1e12 / PEAK_FP32_TFLOPS, 4),
               "ai_flop_per_byte": round(arithmetic_intensity(M, N, K, args.beta), 2),
               "hbm_gbs_at_min_bytes": round(args.batch * min_bytes(M, N, K, args.beta) /
                                             (kern_ms * 1e-3) / 1e9, 1)}
        if args.vendor and args.ops == "NN" and args.batch == 1 and v == -1:
            rec.update(vendor_context(prob, steps, min(args.warmup, steps)))
        print(json.dumps(rec), flush=True)
        del prob
        _torch().cuda.empty_cache()
    return 0


if __name__ == "__main__":
    sys.exit(main())
