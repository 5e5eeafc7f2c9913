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

After timing, the CPU-baseline leg runs the oracle on the host over a row
sample of the same workload and checks the C the timed calls left behind
against it (normalized error, reported as ``max_norm_err``; the run fails
when it exceeds 1e-5).

Other modes (one JSON line per result, not the contract line):
  --sweep            every square size and rectangular shape, auto choice
  --variants         every kernel variant on the 4096^3 problem
  --shape M N K      a single shape (with --variant V to force a variant)
  --profile          only the timed steps, no ceilings or CPU baseline: the
                     command to run under rocprofv3
  --trace-summary    tables from a rocprofv3 kernel trace of the above

Timing in the non-contract modes.  Each record carries two times per call:
``us_launch``, from HIP events around each Python->C launch (what a caller
issuing one call at a time sees, host launch gap included), and
``us_device``, from events around back-to-back replays of a HIP graph that
holds many calls (the device time per call, launch gaps between dependent
kernels included, host overhead excluded).  With ``--cold`` a third,
``us_cold``: the graph cycles through enough copies of the operands (more
than 1 GiB) that each call misses the 256 MB last-level cache.  Below about
50 us only the device figure describes the kernel (Tinyforge README, its
note on benchmark harness errors at small sizes).

Accounting (as on the pages): FLOPs = 2*M*N*K, the epilogue is not counted
("Optimizing SGEMM in CUDA" and "The road to a fast GEMM", section "The
problem and the ceiling"); algorithmic bytes = 4*(M*K + K*N + M*N), plus
4*M*N when beta != 0 (C read and written).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
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
# The largest workspace the workspace entry points can use for any problem.
WS_BYTES = 4096 + (32 << 20)
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


def device_ms_per_call(fn_on, est_ms: float, target_ms: float = 2.0, replays: int = 20,
                       copies: int = 1, mark=None):
    """Device time (ms) per call with the host out of the way.

    fn_on(handle, i) enqueues call i on the stream with that hipStream_t
    handle.  reps calls (about target_ms of device work, at least `copies`)
    are captured into one HIP graph, which is replayed `replays` times back to
    back between two events after a short clock-waking burst; returns (ms per
    call, reps).  mark(handle), if given, is called on the timing stream
    right before the timed replays (a separator for kernel traces)."""
    torch = _torch()
    reps = int(min(4000, max(10, copies, target_ms / max(est_ms, 1e-4))))
    reps = -(-reps // copies) * copies
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(min(copies, 4)):
            fn_on(side.cuda_stream, i)
    side.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for i in range(reps):
            fn_on(side.cuda_stream, i)
    cur = torch.cuda.current_stream()
    g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 0.1:
        g.replay()
        torch.cuda.synchronize()
    if mark is not None:
        mark(cur.cuda_stream)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(cur)
    for _ in range(replays):
        g.replay()
    e1.record(cur)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (reps * replays)
    del g
    return ms, reps


# Separator launches for kernel traces: an empty kernel of `code` workgroups
# is enqueued before each timed phase of job j (code = 16 + 4j + phase; phase
# 0: per-launch event timing, 1: graph replays, 2: end of the job), so a
# rocprofv3 kernel trace of a sweep splits into jobs by these dispatches.
def mark_code(job: int, phase: int) -> int:
    return 16 + 4 * job + phase


def _mark(job, phase):
    import dense_fp32_gemm_sgemm_amd as sg

    def fn(handle):
        assert sg.sgemm_ceiling_empty(mark_code(job, phase), handle) == 0
    return fn


class Problem:
    """Device buffers of one GEMM and a zero-overhead launcher."""

    def __init__(self, M, N, K, alpha=1.0, beta=0.0, seed=0, kind="real", ops="NN", batch=1,
                 copies=1, ws=False):
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
        # With ws: calls go through the workspace entry point, with the
        # largest workspace any problem can use (zero-filled once).
        self.ws = torch.zeros(WS_BYTES, dtype=torch.uint8, device="cuda") if ws else None
        # Further copies of every operand (same values) for cold-cache timing.
        self.sets = [(self.A, self.B, self.C)]
        for _ in range(copies - 1):
            self.sets.append((self.A.clone(), self.B.clone(), self.C.clone()))

    def launcher_on(self, variant=-1):
        """fn(handle, i): one call on stream `handle` with operand copy
        i % copies; raises on a non-zero status."""
        import dense_fp32_gemm_sgemm_amd as sg
        sa, sb, sc = self.strides
        ptrs = [(a.data_ptr(), b.data_ptr(), c.data_ptr()) for a, b, c in self.sets]
        head = (int(self.ta), int(self.tb), self.M, self.N, self.K, float(self.alpha))
        if self.ws is None:
            fn_ex = sg.load().sgemm_strided_batched_ex
            tail = ()
        else:
            fn_ex = sg.load().sgemm_strided_batched_ws_ex
            tail = (self.ws.data_ptr(), WS_BYTES)

        def fn(handle, i=0):
            pa, pb, pc = ptrs[i % len(ptrs)]
            st = fn_ex(*head, pa, self.lda, sa, pb, self.ldb, sb, float(self.beta), pc,
                       max(1, self.N), sc, self.batch, *tail, handle, variant)
            if st != 0:
                raise RuntimeError("sgemm status %d: %s" % (st, sg.sgemm_status_string(st)))
        return fn

    def launcher(self, variant=-1):
        """fn(): one call on the problem's stream."""
        on = self.launcher_on(variant)
        h = self.stream.cuda_stream
        return lambda: on(h)

    def variant_name(self, variant=-1):
        import dense_fp32_gemm_sgemm_amd as sg
        if variant >= 0:
            return sg.sgemm_variant_name(variant)
        sa, sb, sc = self.strides
        args = (int(self.ta), int(self.tb), self.M, self.N, self.K, self.alpha, self.A.data_ptr(),
                self.lda, sa, self.B.data_ptr(), self.ldb, sb, self.beta, self.C.data_ptr(),
                max(1, self.N), sc, self.batch)
        if self.ws is None:
            v = sg.sgemm_strided_batched_select_variant(*args)
        else:
            v = sg.sgemm_strided_batched_ws_select_variant(*args, WS_BYTES)
        return sg.sgemm_variant_name(v) if v >= 0 else "none"


def measure_ceilings(samples: int = 15):
    """Measured FP32 matrix-core and vector rates, HBM copy and read-only
    stream rates, and the dispatch floor."""
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
    del dst
    # Read-only stream over 1 GiB (four times the last-level cache), so every
    # launch reads HBM; the grid is swept and the best kept.
    n2 = 2 * n
    big = torch.ones(n2, dtype=torch.float32, device="cuda")
    del src
    rsink = torch.empty(NUM_CUS * 32 * 256, dtype=torch.float32, device="cuda")
    best = 0.0
    for per_cu in (1, 2, 4, 8, 16, 32):
        # device time per launch (graph replays, as the kernels it is set
        # against are timed), so no host gap lowers the roof; launches read
        # the two 1 GiB halves in turn (each from HBM: the last-level cache
        # holds 256 MB), and 1 GiB streams faster than 2 GiB in one launch
        # (6.5 against 6.0 TB/s)
        def rd(hh, i, per_cu=per_cu):
            assert sg.sgemm_ceiling_read(big.data_ptr() + 4 * n * (i % 2), n, NUM_CUS * per_cu,
                                         rsink.data_ptr(), hh) == 0
        ms, _ = device_ms_per_call(rd, 4 * n / 6e12 * 1e3, target_ms=5.0, replays=samples, copies=2)
        rate = 4 * n / (ms * 1e-3) / 1e9
        if rate > best:
            best, out["hbm_read_grid_per_cu"] = rate, per_cu
    out["hbm_read_gbs"] = best
    out["hbm_read_mib"] = 4 * n >> 20
    del big, rsink
    # Dispatch floor: an empty one-workgroup kernel, back to back in a graph.
    out["dispatch_floor_us"] = device_ms_per_call(lambda hh, i: sg.sgemm_ceiling_empty(1, hh), 0.002,
                                                  target_ms=1.0)[0] * 1e3
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


def cpu_baseline(target_s: float = 12.0, check=None):
    """The oracle (as it stands) on a bounded row sample of the 4096^3
    workload, on the host cores.

    check: optional (C, ncols) -- the GPU's 4096^3 result (numpy float32) and
    a number of whole columns; the rows the oracle timing produced, plus
    `ncols` seeded columns (each crosses every tile row), are compared with C
    and the normalized error max |C - C_ref| / (sum_k |A_ik||B_kj|) is added
    to the record ("check")."""
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
    ref, den = oracle.gemm(A, B, rows=sel)
    dt = time.perf_counter() - t0
    gfl = flops(nrows, HEADLINE.N, HEADLINE.K) / dt / 1e9
    rec = {"value": round(gfl, 3), "unit": "GFLOPS", "cores": oracle.max_threads(),
           "kind": "oracle",
           "sample": "first %d of 4096 output rows of the 4096^3 workload (fp64 i-k-j "
                     "oracle, OpenMP over rows), %.1f s" % (nrows, dt)}
    if check is not None:
        C, ncols = check
        err_r = oracle.normalized_error(C[sel], ref, den)
        cols = np.sort(np.random.default_rng(4096).choice(HEADLINE.N, size=ncols, replace=False))
        cref, cden = oracle.gemm(A, B, cols=cols)
        err_c = oracle.normalized_error(C[:, cols], cref, cden)
        rec["check"] = {"max_norm_err": max(err_r, err_c), "rows": int(nrows), "cols": int(ncols),
                        "what": "the C left by the timed calls against the oracle: the first %d "
                                "whole rows and %d seeded whole columns" % (nrows, ncols)}
    del ref, den
    # The other sizes the oracle is quoted at: all of 256^3, and a row sample
    # of 8192^3 (about a second of CPU time together).
    by_size = {}
    for n, r in ((256, 256), (8192, 128)):
        An, Bn, _ = draw_workload(squares[n])
        t0 = time.perf_counter()
        oracle.gemm(An, Bn, rows=np.arange(r))
        by_size["%d^3 (%d rows)" % (n, r)] = round(flops(r, n, n) / (time.perf_counter() - t0) / 1e9, 3)
        del An, Bn
    rec["by_size"] = by_size
    return rec


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
    strict FP32, timed the same two ways as the library.  A reported
    stopwatch, not part of the library; beta = 0 problems only (torch.mm
    overwrites its output)."""
    torch = _torch()
    if prob.beta != 0.0 or prob.ta or prob.batch != 1:
        return {}
    prev = torch.backends.cuda.matmul.allow_tf32
    torch.backends.cuda.matmul.allow_tf32 = False
    out = {}
    try:
        A, C = prob.A, prob.C
        B = prob.B.t() if prob.tb else prob.B
        fn = lambda: torch.mm(A, B, out=C)
        for _ in range(warmup):
            fn()
        wake(0.1, fn)
        _, per = time_steps(fn, steps, torch.cuda.current_stream())
        ms = statistics.median(per)
        out["torch_mm_us_launch"] = round(ms * 1e3, 2)
        try:
            dev, _ = device_ms_per_call(lambda h, i: fn(), ms)
            out["torch_mm_us_device"] = round(dev * 1e3, 2)
        except Exception as e:  # capture refused: keep the launch figure only
            out["torch_mm_graph_error"] = type(e).__name__
    finally:
        torch.backends.cuda.matmul.allow_tf32 = prev
    best = out.get("torch_mm_us_device", out["torch_mm_us_launch"])
    out["torch_mm_tflops"] = round(flops(prob.M, prob.N, prob.K) / (best * 1e-6) / 1e12, 2)
    return out


def binding_roof(work: float, nbytes: float, us: float, ceil) -> dict:
    """The roof that binds one call: the largest of its floors -- the matrix-
    core time (work at the measured 32x32x2 FP32 rate), the HBM time (the
    algorithmic bytes at the measured read-only stream rate; writes priced as
    reads, which only lowers this floor) and the dispatch floor (an empty
    kernel) -- and the call's fraction of it."""
    t = {"mfma": work / (ceil["mfma_f32_32x32x2_tflops"] * 1e12) * 1e6,
         "hbm": nbytes / (ceil["hbm_read_gbs"] * 1e9) * 1e6}
    if ceil.get("dispatch_floor_us"):
        t["latency"] = ceil["dispatch_floor_us"]
    bound = max(t, key=t.get)
    return {"bound": bound, "frac_of_bound": round(t[bound] / us, 4),
            "floor_us": {k: round(v, 3) for k, v in t.items()},
            "frac_measured_mfma": round(t["mfma"] / us, 4),
            "frac_datasheet": round(work / (us * 1e-6) / 1e12 / PEAK_FP32_TFLOPS, 4)}


DATASHEET_CEILINGS = {"mfma_f32_32x32x2_tflops": PEAK_FP32_TFLOPS, "hbm_read_gbs": PEAK_HBM_GBS,
                      "dispatch_floor_us": None, "source": "datasheet"}


def time_call(prob: Problem, variant: int, steps: int, warmup: int, job: int, cold=False):
    """Times one problem both ways (see the module docstring); with cold,
    also on rotated operand copies (a second Problem with enough copies to
    exceed 1 GiB).  Trace separators mark the phases of `job`."""
    torch = _torch()
    fn = prob.launcher(variant)
    for _ in range(warmup):
        fn()
    wake(0.1, fn)
    h = prob.stream.cuda_stream
    _mark(job, 0)(h)
    _, per = time_steps(fn, steps, prob.stream)
    launch_ms = statistics.median(per)
    dev_ms, reps = device_ms_per_call(prob.launcher_on(variant), launch_ms, mark=_mark(job, 1))
    _mark(job, 2)(h)
    rec = {"job": job, "us_launch": round(launch_ms * 1e3, 3), "us_launch_min": round(min(per) * 1e3, 3),
           "us_device": round(dev_ms * 1e3, 3), "graph_reps": reps, "graph_replays": 20}
    if cold:
        nb = prob.batch * min_bytes(prob.M, prob.N, prob.K, prob.beta)
        copies = int(min(256, -(-1.5 * 2 ** 30 // nb)))
        cp = Problem(prob.M, prob.N, prob.K, prob.alpha, prob.beta, seed=0,
                     ops=("T" if prob.ta else "N") + ("T" if prob.tb else "N"), batch=prob.batch,
                     copies=copies, ws=prob.ws is not None)
        cold_ms, _ = device_ms_per_call(cp.launcher_on(variant), dev_ms, copies=copies)
        rec["us_cold"] = round(cold_ms * 1e3, 3)
        rec["cold_copies"] = copies
        del cp
        torch.cuda.empty_cache()
    return rec


def read_floor(nbytes: float, cold: bool = True, grids=(1, 2, 4, 8, 16)):
    """The read-only stream kernel over `nbytes` (rounded up to 16 bytes):
    device microseconds per launch, best over the grids (workgroups per CU)
    -- warm (one buffer, re-read) or cold (rotated over copies that together
    exceed 1.5 GiB, as the cold GEMM timings are).  The attainable HBM time
    for a call that must stream that many bytes once."""
    torch = _torch()
    import dense_fp32_gemm_sgemm_amd as sg
    n = int(-(-nbytes // 16)) * 4                      # floats, a multiple of 4
    copies = int(min(256, -(-1.5 * 2 ** 30 // (4 * n)))) if cold else 1
    buf = torch.ones(n * copies, dtype=torch.float32, device="cuda")
    sink = torch.empty(NUM_CUS * 16 * 256, dtype=torch.float32, device="cuda")
    best = None
    for per_cu in grids:
        def fn(h, i, per_cu=per_cu):
            assert sg.sgemm_ceiling_read(buf.data_ptr() + 4 * n * (i % copies), n, NUM_CUS * per_cu,
                                         sink.data_ptr(), h) == 0
        ms, _ = device_ms_per_call(fn, 4 * n / 5e12 * 1e3, copies=copies)
        best = ms if best is None else min(best, ms)
    del buf, sink
    torch.cuda.empty_cache()
    return best * 1e3


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
    ap.add_argument("--rows", type=int, nargs="+", metavar="M",
                    help="with --few-rows: only these row counts of the grid")
    ap.add_argument("--nk", type=int, nargs=2, metavar=("N", "K"),
                    help="with --few-rows: only this (N, K) pair of the grid")
    ap.add_argument("--vendor", action="store_true",
                    help="with --sweep/--shape: also time torch.mm in strict FP32 (context only)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true")
    ap.add_argument("--ws", action="store_true",
                    help="non-contract modes: call the workspace entry point (4 KiB + 32 MiB workspace)")
    ap.add_argument("--counters-md", nargs="+", metavar="JSON",
                    help="format --counter-summary outputs of several passes as one markdown table")
    ap.add_argument("--times", nargs="+", metavar="JSONL",
                    help="with --counters-md: timing runs (--sweep / --shapes-from) giving device times")
    ap.add_argument("--sweep-md", nargs="+", metavar="JSONL",
                    help="format a --sweep run (and optionally its --ws run) as a markdown table")
    ap.add_argument("--few-rows-md", metavar="JSONL", help="format a --few-rows run as a markdown table")
    ap.add_argument("--variants-md", nargs="+", metavar="JSONL",
                    help="format --variants / --matrix / --shape runs as a shape x variant table")
    ap.add_argument("--read-floor", action="store_true",
                    help="with --cold: also time the read-only stream kernel over each "
                         "problem's algorithmic bytes, cold (the attainable HBM time at that size)")
    ap.add_argument("--read-ladder", action="store_true",
                    help="time the read-only stream kernel warm and cold over 4 MiB .. 1 GiB")
    ap.add_argument("--cold", action="store_true",
                    help="non-contract modes: also time on rotated operand copies past the 256 MB cache")
    ap.add_argument("--shapes-from", metavar="FILE",
                    help="extra shapes, one 'M N K' per line (with --sweep: added to it)")
    ap.add_argument("--job0", type=int, default=0,
                    help="first job number of the trace separators (to merge several runs)")
    ap.add_argument("--trace-summary", nargs=2, metavar=("KERNEL_TRACE_CSV", "RUN_LOG"),
                    help="print a markdown table of kernel-only times from a rocprofv3 kernel "
                         "trace and the JSON lines of the run it traced (no GPU needed)")
    ap.add_argument("--choice-table", action="store_true",
                    help="every scored tile family on each tile-choice shape (device time)")
    ap.add_argument("--choice-table-md", metavar="RUN_LOG",
                    help="format the JSON lines of a --choice-table run as a markdown table")
    ap.add_argument("--counter-summary", nargs=2, metavar=("COUNTER_CSV", "RUN_LOG"),
                    help="per-job mean counters from a rocprofv3 counter_collection.csv and the "
                         "JSON lines of the run it profiled (no GPU needed)")
    args = ap.parse_args(argv)

    if args.trace_summary:
        sys.stdout.write(trace_summary(*args.trace_summary))
        return 0
    if args.counter_summary:
        for rec in counter_summary(*args.counter_summary):
            print(json.dumps(rec))
        return 0
    if args.counters_md:
        sys.stdout.write(counters_md(args.counters_md, args.times))
        return 0
    if args.sweep_md:
        sys.stdout.write(sweep_md(*args.sweep_md))
        return 0
    if args.variants_md:
        sys.stdout.write(variants_md(args.variants_md))
        return 0
    if args.few_rows_md:
        sys.stdout.write(few_rows_md(args.few_rows_md))
        return 0
    if args.choice_table_md:
        sys.stdout.write(choice_table_md(args.choice_table_md))
        return 0

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
    if args.read_ladder:
        for mib in (4, 16, 64, 256, 1024):
            nb = mib * 2 ** 20
            warm, cold = read_floor(nb, cold=False), read_floor(nb, cold=True)
            print(json.dumps({"mode": "read_ladder", "mib": mib, "us_warm": round(warm, 3),
                              "us_cold": round(cold, 3), "gbs_warm": round(nb / warm / 1e3, 1),
                              "gbs_cold": round(nb / cold / 1e3, 1)}), flush=True)
        return 0
    if args.choice_table:
        return choice_table(args)
    if (args.sweep or args.variants or args.shape or args.profile or args.matrix or args.copy_calib
            or args.shapes_from):
        return run_modes(args)

    M = N = K = 4096
    prob = Problem(M, N, K, 1.0, 0.0, seed=0)
    vname = prob.variant_name(args.variant)
    total, per = bench_problem(prob, args.steps, args.warmup, args.variant)
    ms_step = total / args.steps
    kern_ms = statistics.mean(per)
    value = flops(M, N, K) / (ms_step * 1e-3) / 1e9
    achieved = flops(M, N, K) / (kern_ms * 1e-3) / 1e12
    # The C the timed calls left behind (beta = 0: every call rewrites it).
    torch.cuda.synchronize()
    timed_c = prob.C.cpu().numpy()

    clocks = None if args.no_ceilings else clock_under_load(prob.launcher(args.variant))
    ceilings = None if args.no_ceilings else measure_ceilings()
    cpu = None if args.no_cpu_baseline else cpu_baseline(check=(timed_c, 256))
    traffic = stored_traffic(vname)
    check = cpu.pop("check") if cpu else None

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
        "max_norm_err": None if check is None else float("%.4g" % check["max_norm_err"]),
        "check": check,
        "gpu_clocks": clocks,
    }
    if ceilings:
        mf = ceilings["mfma_f32_32x32x2_tflops"]
        line["measured_ceilings"] = {k: round(v, 2) for k, v in ceilings.items()}
        line["pct_of_measured_mfma_f32"] = round(100.0 * value / 1e3 / mf, 2)
        # above 100: the matrix cores outrun unpacked v_fma_f32 (packed FP32
        # vector instructions are switched off in the library's compile flags)
        line["pct_of_measured_valu_f32"] = round(100.0 * value / 1e3 / ceilings["valu_fma_f32_tflops"], 2)
        line["pct_of_datasheet_fp32"] = round(100.0 * value / 1e3 / PEAK_FP32_TFLOPS, 2)
    print(json.dumps(line), flush=True)
    if check is not None and not check["max_norm_err"] <= 1e-5:
        print("bench: timed 4096^3 result fails the oracle check (normalized error %.3g > 1e-5)"
              % check["max_norm_err"], file=sys.stderr)
        return 3
    return 0


FEW_ROWS_M = (1, 4, 8, 12, 16, 20, 24, 32)
FEW_ROWS_NK = ((4096, 4096), (8192, 8192), (16384, 16384), (1024, 4096), (2048, 2048),
               (4096, 1024), (4096, 16384), (65536, 1024), (1024, 16384))


def few_rows(args):
    """Per shape and orientation of B: the automatic choice, each few-rows
    candidate forced (vector-unit kernel, split-K 64x64 tiles, matrix-core
    kernel) and torch.mm in strict FP32, each timed per launch and on the
    device (graph replays); the automatic choice also cold."""
    import dense_fp32_gemm_sgemm_amd as sg
    torch = _torch()
    names = sg.variant_names()
    cands = [names.index(n) for n in ("skinny_m8", "mfma16_64x64x64_4x2_pipe_splitk", "fewrows_m32")]
    ceil = _sweep_ceilings(args)
    job = args.job0
    for M in (args.rows or FEW_ROWS_M):
        for N, K in ([tuple(args.nk)] if args.nk else FEW_ROWS_NK):
            for ops in ("NN", "NT"):
                prob = Problem(M, N, K, ops=ops)
                rec = {"mode": "few-rows", "M": M, "N": N, "K": K, "ops": ops,
                       "auto": prob.variant_name(-1), "jobs": {}}
                for v in [-1] + cands:
                    key = "auto" if v < 0 else names[v]
                    t = time_call(prob, v, args.steps, min(args.warmup, args.steps), job,
                                  cold=(v < 0 and args.cold))
                    rec["jobs"][key] = job
                    job += 1
                    rec["us_launch_" + key] = t["us_launch"]
                    rec["us_device_" + key] = t["us_device"]
                    rec["reps_" + key] = t["graph_reps"]
                    if "us_cold" in t:
                        rec["us_cold_auto"] = t["us_cold"]
                if args.ws:
                    # the workspace entry point's automatic choice (timed only
                    # where it differs from the plain one)
                    pw = Problem(M, N, K, ops=ops, ws=True)
                    rec["auto_ws"] = pw.variant_name(-1)
                    if rec["auto_ws"] != rec["auto"]:
                        t = time_call(pw, -1, args.steps, min(args.warmup, args.steps), job, cold=args.cold)
                        rec["jobs"]["auto_ws"] = job
                        job += 1
                        rec["us_device_auto_ws"] = t["us_device"]
                        if "us_cold" in t:
                            rec["us_cold_auto_ws"] = t["us_cold"]
                    del pw
                nb = min_bytes(M, N, K)
                rec["auto_gbs_device"] = round(nb / (rec["us_device_auto"] * 1e-6) / 1e9, 1)
                if "us_cold_auto" in rec:
                    rec["auto_gbs_cold"] = round(nb / (rec["us_cold_auto"] * 1e-6) / 1e9, 1)
                rec.update(binding_roof(flops(M, N, K), nb, rec.get("us_cold_auto", rec["us_device_auto"]),
                                        ceil))
                rec.update(vendor_context(prob, args.steps, min(args.warmup, args.steps)))
                print(json.dumps(rec), flush=True)
                del prob
                torch.cuda.empty_cache()
    return 0


def _sweep_ceilings(args):
    if args.no_ceilings:
        return DATASHEET_CEILINGS
    c = measure_ceilings(samples=7)
    c["source"] = "measured"
    print(json.dumps({"mode": "ceilings", **{k: (round(v, 3) if isinstance(v, float) else v)
                                              for k, v in c.items()}}), flush=True)
    return c


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
        # only timed calls (no graph, no ceilings): the command to run under
        # rocprofv3; several shapes (--shapes-from) are split by separators
        if args.shapes_from:
            with open(args.shapes_from) as f:
                shapes = [tuple(int(x) for x in line.split()[:3]) for line in f
                          if line.strip() and not line.startswith("#")]
        else:
            shapes = [tuple(args.shape) if args.shape else (4096, 4096, 4096)]
        for j, shape in enumerate(shapes):
            # with --cold the calls cycle through copies of the operands that
            # together exceed 1.5 GiB (each call reads its operands from HBM)
            nb = args.batch * min_bytes(*shape, args.beta)
            copies = int(min(256, -(-1.5 * 2 ** 30 // nb))) if args.cold else 1
            prob = Problem(*shape, args.alpha, args.beta, seed=0, ops=args.ops, batch=args.batch,
                           ws=args.ws, copies=copies)
            fn_on, h0, turn = prob.launcher_on(args.variant), prob.stream.cuda_stream, [0]

            def fn(fn_on=fn_on, h0=h0, turn=turn):
                fn_on(h0, turn[0])
                turn[0] += 1
            for _ in range(args.warmup):
                fn()
            torch_ = _torch()
            wake(0.1, fn)  # clocks up before the timed calls
            torch_.cuda.synchronize()
            _mark(args.job0 + j, 1)(prob.stream.cuda_stream)
            _, per = time_steps(fn, args.steps, prob.stream)
            _mark(args.job0 + j, 2)(prob.stream.cuda_stream)
            kern_ms = statistics.mean(per)
            print(json.dumps({"mode": "profile", "job": args.job0 + j, "M": shape[0], "N": shape[1],
                              "K": shape[2], "ops": args.ops, "batch": args.batch, "copies": copies,
                              "variant": prob.variant_name(args.variant), "steps": args.steps,
                              "graph_reps": args.steps, "graph_replays": 1,
                              "us_device": round(kern_ms * 1e3, 3), "us_launch": round(kern_ms * 1e3, 3),
                              "kernel_ms_mean": round(kern_ms, 5),
                              "tflops": round(args.batch * flops(*shape) / (kern_ms * 1e-3) / 1e12, 2)}),
                  flush=True)
            del prob
            torch_.cuda.empty_cache()
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
    if args.shapes_from:
        with open(args.shapes_from) as f:
            extra = [tuple(int(x) for x in line.split()[:3]) for line in f
                     if line.strip() and not line.startswith("#")]
        jobs = [(sh, args.variant) for sh in extra] if not (args.sweep or args.matrix) else jobs + [
            (sh, -1) for sh in extra]
    ceil = _sweep_ceilings(args)
    mode = "sweep" if args.sweep else ("matrix" if args.matrix else "variant")
    for j, (shape, v) in enumerate(jobs):
        M, N, K = shape
        prob = Problem(M, N, K, args.alpha, args.beta, seed=0, ops=args.ops, batch=args.batch,
                       ws=args.ws)
        name = prob.variant_name(v)
        work = flops(M, N, K) * args.batch
        nb = args.batch * min_bytes(M, N, K, args.beta)
        steps = max(5, min(args.steps, int(2e12 / max(work, 1.0))))
        if name == "simple" and work > 1e11:
            steps = 3
        cold = args.cold and nb >= 4e6
        t = time_call(prob, v, steps, min(args.warmup, steps), args.job0 + j, cold=cold)
        us = t["us_device"]
        rec = {"mode": mode, "ops": args.ops, "batch": args.batch, "M": M, "N": N, "K": K,
               "beta": args.beta, "variant": name, "forced": v >= 0, "workspace": bool(args.ws), "steps": steps,
               **t,
               "tflops_device": round(work / (us * 1e-6) / 1e12, 3),
               "tflops_launch": round(work / (t["us_launch"] * 1e-6) / 1e12, 3),
               "ai_flop_per_byte": round(work / nb, 2),
               "hbm_gbs_device": round(nb / (us * 1e-6) / 1e9, 1)}
        if "us_cold" in t:
            rec["hbm_gbs_cold"] = round(nb / (t["us_cold"] * 1e-6) / 1e9, 1)
            if args.read_floor:
                # the read-only stream over the same bytes, cold: what any
                # kernel that reads them once can reach at this size
                rec["us_read_cold"] = round(read_floor(nb, cold=True), 3)
                rec["frac_of_read_cold"] = round(rec["us_read_cold"] / t["us_cold"], 4)
        # rated on the cold time where the bytes bind, else the warm one
        roof = binding_roof(work, nb, us, ceil)
        if roof["bound"] == "hbm" and "us_cold" in t:
            roof = binding_roof(work, nb, t["us_cold"], ceil)
            roof["rated_on"] = "us_cold"
        rec.update(roof)
        if args.vendor and args.batch == 1 and v == -1:
            rec.update(vendor_context(prob, steps, min(args.warmup, steps)))
        print(json.dumps(rec), flush=True)
        del prob
        _torch().cuda.empty_cache()
    return 0


# The tile families the automatic choice scores, with their tile sizes and
# whether they also run fewer rows than the tile (A untransposed); the tail
# forms need the workspace entry point.
CHOICE_FAMILIES = (
    ("256x256", "mfma32_256x256x32_2x2_sched", 256, 256, False),
    ("128x128 w4", "mfma16_128x128x32_2x2_sched", 128, 128, False),
    ("128x128 w8", "mfma16_128x128x64_4x2_sched", 128, 128, False),
    ("128x64", "mfma16_128x64x64_4x2_sched", 128, 64, False),
    ("64x64", "mfma16_64x64x64_4x2_sched", 64, 64, False),
    ("64x64 split-K", "mfma16_64x64x64_4x2_sched_splitk", 64, 64, False),
    ("32x64", "mfma16_32x64x64_2x2_sched", 32, 64, True),
    ("32x64 split-K", "mfma16_32x64x64_2x2_sched_splitk", 32, 64, True),
    ("128x128 w4 tail", "mfma16_128x128x32_2x2_sched_tail", 128, 128, False),
    ("128x128 w8 tail", "mfma16_128x128x64_4x2_sched_tail", 128, 128, False),
    ("128x64 tail", "mfma16_128x64x64_4x2_sched_tail", 128, 64, False),
    ("64x64 tail", "mfma16_64x64x64_4x2_sched_tail", 64, 64, False),
    ("edge split", "edge_split", 1, 1, False),
)


def has_thin_edge(M, N, K):
    """Whether the library's edge split applies: K of about 1024 or more and
    a dimension that overruns some tile family's tiles by a thin edge of 1
    to 32 (rows: tiles of 256, 128, 64 or 32; columns: 256, 128 or 64)."""
    if K < 1000:
        return False
    return (any(M > t and 1 <= M % t <= 32 for t in (256, 128, 64, 32)) or
            any(N > t and 1 <= N % t <= 32 for t in (256, 128, 64)))


def choice_table(args):
    """Every scored tile family (device time, graph replays) on each shape of
    workloads.TILE_CHOICE_SHAPES, with the automatic choices of the plain and
    the workspace entry points: one JSON line per shape."""
    import dense_fp32_gemm_sgemm_amd as sg
    from workloads import TILE_CHOICE_SHAPES
    torch = _torch()
    names = sg.variant_names()
    for M, N, K, ops in TILE_CHOICE_SHAPES:
        prob = Problem(M, N, K, ops=ops, ws=True)
        rec = {"mode": "choice", "M": M, "N": N, "K": K, "ops": ops, "tflops": {}}
        for label, vname, bm, bn, short_m in CHOICE_FAMILIES:
            if not ((M >= bm or (short_m and ops[0] == "N")) and N >= bn):
                continue  # the family's loop does not run this shape
            if vname == "edge_split" and not has_thin_edge(M, N, K):
                continue  # (it would run the automatic choice whole)
            v = names.index(vname)
            fn = prob.launcher(v)
            fn()
            fn()
            _, per = time_steps(fn, 3, prob.stream)
            ms, _ = device_ms_per_call(prob.launcher_on(v), min(per), replays=10)
            rec["tflops"][label] = round(flops(M, N, K) / (ms * 1e-3) / 1e12, 2)
        rec["auto_ws"] = prob.variant_name(-1)
        prob.ws = None
        rec["auto"] = prob.variant_name(-1)
        print(json.dumps(rec), flush=True)
        del prob
        torch.cuda.empty_cache()
    return 0


def _current_choices(M, N, K, ops):
    """(plain, workspace) automatic choices of the built library for a shape
    (host-only queries; no GPU needed)."""
    import dense_fp32_gemm_sgemm_amd as sg
    ta, tb = int(ops[0] == "T"), int(ops[1] == "T")
    lda, ldb, f = (M if ta else K), (K if tb else N), 256
    v = sg.sgemm_strided_batched_select_variant(ta, tb, M, N, K, 1.0, f, lda, 0, f, ldb, 0, 0.0, f, N,
                                                0, 1)
    w = sg.sgemm_strided_batched_ws_select_variant(ta, tb, M, N, K, 1.0, f, lda, 0, f, ldb, 0, 0.0, f,
                                                   N, 0, 1, WS_BYTES)
    return sg.sgemm_variant_name(v), sg.sgemm_variant_name(w)


def choice_table_md(log_path: str) -> str:
    """The --choice-table JSON lines as a markdown table (best family bold);
    the two choice columns are those of the library as built now."""
    labels = [f[0] for f in CHOICE_FAMILIES]
    short = {f[1]: f[0] for f in CHOICE_FAMILIES}
    out = ["| M x N x K | ops | " + " | ".join(labels) + " | auto | auto with workspace |",
           "|---|---|" + "---|" * len(labels) + "---|---|"]
    with open(log_path) as f:
        for line in f:
            if not line.startswith("{"):
                continue
            r = json.loads(line)
            if r.get("mode") != "choice":
                continue
            t = r["tflops"]
            best = max(t.values()) if t else None
            cells = []
            for lab in labels:
                if lab not in t:
                    cells.append("-")
                elif t[lab] == best:
                    cells.append("**%.1f**" % t[lab])
                else:
                    cells.append("%.1f" % t[lab])
            auto, auto_ws = _current_choices(r["M"], r["N"], r["K"], r["ops"])
            out.append("| %dx%dx%d | %s | %s | %s | %s |" % (
                r["M"], r["N"], r["K"], r["ops"], " | ".join(cells), short.get(auto, auto),
                short.get(auto_ws, auto_ws)))
    return "\n".join(out) + "\n"


def _jsonl(path: str, mode=None) -> list:
    out = []
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line.startswith("{"):
                r = json.loads(line)
                if mode is None or r.get("mode") == mode:
                    out.append(r)
    return out


def sweep_md(sweep_path: str, ws_path: str = None) -> str:
    """A --sweep run (with --cold, --vendor, --read-floor) as a markdown
    table: device time per call, launch-inclusive time, cold time, the
    binding roof and the fraction of it, the same-size cold read floor, the
    vendor stopwatch; with ws_path the workspace entry point's run beside."""
    ceil = (_jsonl(sweep_path, "ceilings") or [{}])[0]
    ws = {(r["M"], r["N"], r["K"]): r for r in _jsonl(ws_path, "sweep")} if ws_path else {}
    out = []
    if ceil:
        out.append("Measured ceilings of this run: MFMA 32x32x2 %.1f TFLOP/s, 16x16x4 %.1f, v_fma_f32 %.1f; "
                   "HBM read-only stream %.0f GB/s (%s), copy %.0f GB/s; dispatch floor %.2f us.\n"
                   % (ceil["mfma_f32_32x32x2_tflops"], ceil["mfma_f32_16x16x4_tflops"],
                      ceil["valu_fma_f32_tflops"], ceil["hbm_read_gbs"],
                      "%d MiB per launch, cold" % ceil["hbm_read_mib"] if "hbm_read_mib" in ceil
                      else "2 GiB", ceil["hbm_copy_gbs"], ceil["dispatch_floor_us"]))
    head = ("| M x N x K | variant | device us | TFLOP/s | launch us | cold us | bound | floor us | "
            "frac of bound | frac of datasheet | read floor cold us | vendor device us | vendor / ours |")
    if ws:
        head += " workspace variant | ws device us | ws TFLOP/s | ws cold us |"
    out += [head, "|" + "---|" * (head.count("|") - 1)]
    for r in _jsonl(sweep_path, "sweep"):
        key = (r["M"], r["N"], r["K"])
        floor = r["floor_us"][r["bound"]]
        vend = r.get("torch_mm_us_device")
        row = "| %dx%dx%d | %s | %.2f | %.2f | %.2f | %s | %s%s | %.2f | %.3f | %.3f | %s | %s | %s |" % (
            key + (r["variant"], r["us_device"], r["tflops_device"], r["us_launch"],
                   "%.2f" % r["us_cold"] if "us_cold" in r else "-", r["bound"],
                   " (cold)" if r.get("rated_on") == "us_cold" else "", floor, r["frac_of_bound"],
                   r["frac_datasheet"], "%.2f" % r["us_read_cold"] if "us_read_cold" in r else "-",
                   "%.2f" % vend if vend else "-",
                   "%.2f" % (vend / r["us_device"]) if vend else "-"))
        if ws:
            w = ws.get(key)
            row += (" %s | %.2f | %.2f | %s |" % (w["variant"], w["us_device"], w["tflops_device"],
                                                   "%.2f" % w["us_cold"] if "us_cold" in w else "-") if w
                    else " - | - | - | - |")
        out.append(row)
    return "\n".join(out) + "\n"


def variants_md(paths) -> str:
    """Timing records of --variants / --matrix / --shape / --sweep runs as a
    shape x variant table of TFLOP/s (device time per call), with the
    automatic choice (records not forced) in the last columns; the best
    forced variant of each row in bold."""
    rows, names = {}, []
    for path in paths:
        for r in _jsonl(path):
            if "us_device" not in r or "M" not in r:
                continue
            key = (r.get("batch", 1), r["M"], r["N"], r["K"], r.get("ops", "NN"))
            d = rows.setdefault(key, {"forced": {}, "auto": None})
            if r.get("forced", True) and r.get("mode") != "sweep":
                d["forced"][r["variant"]] = r["tflops_device"]
                if r["variant"] not in names:
                    names.append(r["variant"])
            else:
                d["auto"] = (r["variant"], r["tflops_device"])
    out = ["| batch x M x N x K | ops | " + " | ".join(names) + " | auto | auto TFLOP/s | auto / best |",
           "|---|---|" + "---|" * len(names) + "---|---|---|"]
    for key in sorted(rows, key=lambda k: (k[4], k[0] * k[1] * k[2] * k[3], k)):
        d = rows[key]
        best = max(d["forced"].values()) if d["forced"] else None
        cells = []
        for n in names:
            v = d["forced"].get(n)
            cells.append("-" if v is None else ("**%.2f**" % v if v == best else "%.2f" % v))
        a = d["auto"]
        out.append("| %s%dx%dx%d | %s | %s | %s | %s | %s |" % (
            "%d x " % key[0] if key[0] != 1 else "", key[1], key[2], key[3], key[4], " | ".join(cells),
            a[0] if a else "-", "%.2f" % a[1] if a else "-",
            "%.3f" % (a[1] / best) if a and best else "-"))
    return "\n".join(out) + "\n"


def few_rows_md(path: str) -> str:
    """A --few-rows run as a markdown table of device times (graph replays),
    with the cold time of the automatic choice(s) and the vendor stopwatch."""
    out = ["| M x N x K | B | auto | auto us | auto cold us | cold GB/s | skinny_m8 | pipe_splitk | "
           "fewrows_m32 | workspace auto | ws us | ws cold us | vendor us | vendor / best auto |",
           "|---|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    ratios = []
    for r in _jsonl(path, "few-rows"):
        d = lambda k: r.get("us_device_" + k)
        auto_ws = r.get("auto_ws", r["auto"])
        best = min(x for x in (d("auto"), r.get("us_device_auto_ws")) if x)
        vend = r.get("torch_mm_us_device")
        if vend:
            ratios.append(vend / best)
        out.append("| %dx%dx%d | %s | %s | %.2f | %s | %s | %.2f | %.2f | %.2f | %s | %s | %s | %s | %s |" % (
            r["M"], r["N"], r["K"], r["ops"], r["auto"], d("auto"),
            "%.2f" % r["us_cold_auto"] if "us_cold_auto" in r else "-",
            "%.0f" % r["auto_gbs_cold"] if "auto_gbs_cold" in r else "-",
            d("skinny_m8"), d("mfma16_64x64x64_4x2_pipe_splitk"), d("fewrows_m32"),
            auto_ws if auto_ws != r["auto"] else "(same)",
            "%.2f" % r["us_device_auto_ws"] if "us_device_auto_ws" in r else "-",
            "%.2f" % r["us_cold_auto_ws"] if "us_cold_auto_ws" in r else "-",
            "%.2f" % vend if vend else "-", "%.2f" % (vend / best) if vend else "-"))
    if ratios:
        g = math.exp(sum(math.log(x) for x in ratios) / len(ratios))
        out.append("")
        out.append("Vendor time / best automatic choice (device time): geometric mean %.3f over %d shapes; "
                   "%d below 0.9, %d above 1.1." % (g, len(ratios), sum(x < 0.9 for x in ratios),
                                                   sum(x > 1.1 for x in ratios)))
    return "\n".join(out) + "\n"


def counters_md(paths, times_path=None, copy_fetch_scale=2.0, clock_ghz=2.38) -> str:
    """The --counter-summary outputs of several passes over the same jobs
    (one JSON list per pass) as one markdown table per job: matrix-core busy
    (the deterministic busy count against the profiled dispatch's cycles,
    and against the unprofiled device time when a --sweep / --shapes-from
    run gives it), HBM-side bytes against the algorithmic ones, L2 hit rate,
    LDS bank conflicts."""
    jobs = {}
    for path in paths:
        with open(path) as f:
            text = f.read().strip()
        recs = json.loads(text) if text.startswith("[") else [json.loads(l) for l in text.splitlines() if l]
        for r in recs:
            d = jobs.setdefault(r["job"], {"M": r["M"], "N": r["N"], "K": r["K"], "variant": r["variant"],
                                           "c": {}})
            d["c"].update(r["counters"])
    dev = {}
    for tp in ([times_path] if isinstance(times_path, str) else (times_path or [])):
        for r in _jsonl(tp):
            if "us_device" in r and "M" in r:
                dev[(r["M"], r["N"], r["K"], r.get("variant"))] = r["us_device"]
    out = ["| M x N x K | variant | MFMA busy (profiled) | device us | MFMA busy (device time) | "
           "fetch MB | reads MB (A+B) | fetch / reads | write MB | C MB | L2 hit | LDS conflict cycles |",
           "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for job in sorted(jobs):
        d = jobs[job]
        M, N, K, c = d["M"], d["N"], d["K"], d["c"]
        ideal = c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (4 * NUM_CUS)  # cycles per SIMD
        cyc = c.get("GRBM_GUI_ACTIVE", 0.0) / 8                            # per XCD
        us = dev.get((M, N, K, d["variant"]))
        fetch = c.get("FETCH_SIZE", 0.0) * 1024 * copy_fetch_scale / 1e6
        write = c.get("WRITE_SIZE", 0.0) * 1024 / 1e6
        reads = 4.0 * (M * K + K * N) / 1e6
        cmb = 4.0 * M * N / 1e6
        hit, miss = c.get("TCC_HIT_sum"), c.get("TCC_MISS_sum")
        conf, act = c.get("SQ_LDS_BANK_CONFLICT"), c.get("SQ_LDS_IDX_ACTIVE")
        out.append("| %dx%dx%d | %s | %s | %s | %s | %.1f | %.1f | %.2f | %.1f | %.1f | %s | %s |" % (
            M, N, K, d["variant"], "%.1f%%" % (100 * ideal / cyc) if cyc else "-",
            "%.2f" % us if us else "-", "%.1f%%" % (100 * ideal / (us * 1e3 * clock_ghz)) if us else "-",
            fetch, reads, fetch / reads if reads else 0.0, write, cmb,
            "%.1f%%" % (100 * hit / (hit + miss)) if hit is not None and miss is not None else "-",
            "%.1f%%" % (100 * conf / act) if conf is not None and act else "-"))
    return "\n".join(out) + "\n"


def trace_summary(trace_csv: str, log_path: str, title: str = "") -> str:
    """Markdown table of kernel-only time per call, from a rocprofv3 kernel
    trace (csv) of a --sweep / --shape / --few-rows run and the JSON lines
    that run printed: the dispatches between a job's graph-phase separators
    are that job's graph replays (graph_reps x graph_replays calls)."""
    import csv
    with open(trace_csv) as f:
        rows = list(csv.DictReader(f))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    recs = {}
    with open(log_path) as f:
        for line in f:
            line = line.strip()
            if not line.startswith("{"):
                continue
            r = json.loads(line)
            if "job" in r:
                recs[r["job"]] = r
            for key, j in r.get("jobs", {}).items():
                recs[j] = dict(r, variant=(r["auto"] if key == "auto" else key), job=j,
                               us_device=r["us_device_" + key], us_launch=r["us_launch_" + key],
                               graph_reps=r["reps_" + key], graph_replays=20)
    per_job = {}
    cur = None
    for r in rows:
        name = r["Kernel_Name"]
        if "empty_kernel" in name:
            wg = max(1, int(r.get("Workgroup_Size_X") or r.get("Workgroup_Size") or 64))
            code = int(r.get("Grid_Size_X") or r.get("Grid_Size")) // wg
            job, phase = divmod(code - 16, 4)
            cur = job if phase == 1 else None
            continue
        if cur is None:
            continue
        d = per_job.setdefault(cur, {"ns": 0, "n": 0, "kernels": {}})
        d["ns"] += int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        d["n"] += 1
        short = name.split("(")[0].replace("void ", "")
        d["kernels"][short] = d["kernels"].get(short, 0) + 1
    out = []
    if title:
        out.append(title)
        out.append("")
    out.append("| job | M x N x K | ops | variant | dispatches / call | kernel-only us | "
               "graph us | launch us | TFLOP/s (kernel-only) |")
    out.append("|---|---|---|---|---|---|---|---|---|")
    for job in sorted(per_job):
        r = recs.get(job)
        if r is None:
            continue
        calls = r["graph_reps"] * r["graph_replays"]
        d = per_job[job]
        if not calls:
            continue
        us = d["ns"] / calls / 1e3
        work = flops(r["M"], r["N"], r["K"]) * r.get("batch", 1)
        out.append("| %d | %dx%dx%d | %s | %s | %.2f | %.2f | %.2f | %.2f | %.1f |" % (
            job, r["M"], r["N"], r["K"], r.get("ops", "NN"), r["variant"], d["n"] / calls, us,
            r["us_device"], r["us_launch"], work / (us * 1e-6) / 1e12))
    return "\n".join(out) + "\n"


def counter_summary(counter_csv: str, log_path: str) -> list:
    """Per job of a traced run (--profile / --sweep): each counter summed
    over the GEMM dispatches of a call (a call can launch two kernels, as
    the edge split does) and averaged over the job's timed calls
    (separators and C-scaling launches left out), from a rocprofv3
    counter_collection.csv."""
    import csv
    with open(counter_csv) as f:
        rows = list(csv.DictReader(f))
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    recs = {}
    with open(log_path) as f:
        for line in f:
            line = line.strip()
            if line.startswith("{"):
                r = json.loads(line)
                if "job" in r:
                    recs[r["job"]] = r
    cur, per = None, {}
    seen = set()
    for r in rows:
        name = r["Kernel_Name"]
        if "empty_kernel" in name:
            if r["Dispatch_Id"] in seen:
                continue
            seen.add(r["Dispatch_Id"])
            wg = max(1, int(r.get("Workgroup_Size_X") or r.get("Workgroup_Size") or 64))
            code = int(r.get("Grid_Size_X") or r.get("Grid_Size")) // wg
            job, phase = divmod(code - 16, 4)
            cur = job if phase == 1 else None
            continue
        if cur is None or "scale_kernel" in name:
            continue
        d = per.setdefault(cur, {"kernel": name, "kernels": [], "vals": {}, "dispatches": set()})
        d["dispatches"].add(r["Dispatch_Id"])
        if name not in d["kernels"]:
            d["kernels"].append(name)
        d["vals"].setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    out = []
    for job in sorted(per):
        r = recs.get(job, {})
        d = per[job]
        calls = int(r.get("steps") or len(d["dispatches"]))
        out.append({"job": job, "M": r.get("M"), "N": r.get("N"), "K": r.get("K"),
                    "variant": r.get("variant"), "kernel": d["kernel"], "kernels": d["kernels"],
                    "dispatches": len(d["dispatches"]), "calls": calls,
                    "counters": {k: sum(v) / calls for k, v in d["vals"].items()}})
    return out


if __name__ == "__main__":
    sys.exit(main())
