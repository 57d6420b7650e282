#!/usr/bin/env python3
"""Benchmark of the MX quantize-and-GEMM hot path on one MI355X.

Headline step (the workload the metric is quoted on): the MXFP6 (E2M3,
FLOOR scales, Hadamard-32 along K) linear at the Flux-12B attention
projection shape -- X [4096, 3072] ~N(0,1), W [3072, 3072] ~N(0,0.02),
dY [4096, 3072] ~N(0,1), bf16 -- one step = dual (row + column) packs of X,
W and dY, then forward Y = X W^T, dgrad dX = dY W and wgrad dW = dY^T X
(K = 4096 tokens), bf16 outputs.  value = 3 * 2*M*N*K / step time
(TFLOP/s), inputs resident in HBM; four copies of the inputs are rotated so
that a step does not find its inputs in the 256 MB Infinity Cache.

The same JSON line carries the per-kernel times (HIP events on the stream
the kernels run on), the roofline of the dominant kernel (the GEMM), the
CPU oracle timed on a bounded sample, and -- unless --extra none -- the
other workloads of the metric: the 256^3 MXFP4 parity GEMM, the fused
MXFP6 MLP at M=8192 (3072 -> 12288 -> 3072), the MXFP4 sweep over the five
Flux-12B block linears at M=16384 and the MXFP8 grouped SwiGLU MLP
(G=8, D=2048, F=768, R=32768).

The timed steps replay a captured HIP graph of four consecutive steps (one
per input copy; --no-graph: eager launches).  A step is two launches:
mx_quantize_many packs X, W and dY, mx_gemm_many computes the three GEMMs.
Per-launch
device durations come from HIP events around replays of a graph of ten
back-to-back copies of each launch.

    python bench.py [--gpus 1] [--steps 100] [--warmup 10] [--extra all|none] [--no-cpu-baseline] [--no-graph]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

METRIC = "MX GEMM TFLOP/s and % of MXFP4/6/8 MFMA peak (Flux-12B shapes); quantizer GB/s"
# HBM traffic per launch from the rocprofv3 FETCH_SIZE / WRITE_SIZE counters
# (scaled by what they read for a plain copy), valid while the kernel
# sources are those the counters were taken with
GEMM_TRAFFIC = {"bytes_per_launch": 236.8e6,
                "sources": ("mx_gemm.hip", "mx_device.h", "mx_kernels.h", "mx_tuned.inc"),
                "sources_sha1": "53ce50b65db16e6a151cb803a2fc01e9948211ee"}
# VALU wavefront-instructions per launch of the fused pack (rocprofv3
# SQ_INSTS_VALU), valid while the pack sources are those it was counted with
PACK_VALU = {"instructions_per_launch": 1.028e7, "sources": ("mx_pack.hip", "mx_device.h", "mx_kernels.h"),
             "sources_sha1": "2945333d2cfbd4699be5771f3ec74b31d38e2639"}
# peak VALU issue: 256 CUs x 4 SIMDs x 2.4 GHz, two wave64 instructions per
# four cycles on each SIMD (gfx950 issues two VALU instructions of different
# wavefronts together), i.e. the chip's 157.3 TFLOP/s of fp32 vector FMA
# counted in wave64 instructions (G wavefront-instructions per second)
VALU_PEAK_GIPS = 256 * 4 * 2.4 * 2 / 4
PACK_TRAFFIC = {"bytes_per_launch": 123.5e6, "sources": ("mx_pack.hip", "mx_device.h", "mx_kernels.h"),
                "sources_sha1": "2945333d2cfbd4699be5771f3ec74b31d38e2639"}


def measured_traffic(rec):
    """rec's traffic if its kernel sources are unchanged since, else None."""
    import hashlib
    h = hashlib.sha1()
    for f in rec["sources"]:
        with open(os.path.join(ROOT, "microscaling_block_scaled_mx_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    key = "bytes_per_launch" if "bytes_per_launch" in rec else "instructions_per_launch"
    return rec[key] if h.hexdigest() == rec["sources_sha1"] else None


PEAK_TFLOPS = {"fp4": 10100.0, "fp6": 10100.0, "fp8": 5000.0}  # MI355X dense MFMA
HBM_GBS = 8000.0
# algorithmic bytes per element of a pack: 2 B bf16 in + (bits/8 + 1/32) per output axis
PACK_OUT = {4: 0.5 + 1 / 32, 6: 0.75 + 1 / 32, 8: 1.0 + 1 / 32}


def alu_roofline(pack_us):
    """The fused pack against the VALU issue roofline: the counted VALU
    wavefront-instructions per launch over the launch time, against the
    chip's issue peak.  None when the pack sources changed since the count."""
    n = measured_traffic(PACK_VALU)
    if n is None:
        return None
    achieved = n / (pack_us * 1e-6) / 1e9
    return {"bound": "alu", "achieved": round(achieved, 1), "peak": VALU_PEAK_GIPS,
            "unit": "G wavefront-instructions/s", "frac": round(achieved / VALU_PEAK_GIPS, 4),
            "valu_instructions_per_launch": n}


def dev(a):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda()
    return torch.from_numpy(a).cuda()


class Timer:
    """Per-launch HIP events on the current stream, aggregated by name."""

    def __init__(self):
        self.rec = []
        self.on = False

    def run(self, name, fn, *a, **kw):
        import torch
        if not self.on:
            return fn(*a, **kw)
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        out = fn(*a, **kw)
        e.record()
        self.rec.append((name, s, e))
        return out

    def summary(self):
        import torch
        torch.cuda.synchronize()
        agg = {}
        for name, s, e in self.rec:
            agg.setdefault(name, []).append(s.elapsed_time(e) * 1e3)  # us
        self.rec = []
        return {k: float(np.mean(v)) for k, v in agg.items()}


# ------------------------------------------------------------------ headline: MX linear
class LinearStep:
    def __init__(self, mx, M, N, K, fmt, mode, had, seed, copies=4, rng_inputs=None):
        from microscaling_block_scaled_mx_amd import inputs as I
        import torch
        self.mx, self.M, self.N, self.K, self.fmt, self.mode, self.had = mx, M, N, K, fmt, mode, had
        X, W, dY = rng_inputs if rng_inputs is not None else I.linear(seed, M, N, K)
        self.host = (X, W, dY)
        self.inp = [(dev(X), dev(W), dev(dY)) for _ in range(copies)]
        P = lambda r, k: mx.alloc_packed(r, k, fmt)
        self.Xr, self.Xc, self.Wr, self.Wc, self.dYr, self.dYc = P(M, K), P(K, M), P(N, K), P(K, N), P(M, N), P(N, M)
        e16 = lambda *s: torch.empty(s, dtype=torch.int16, device="cuda")
        self.Y, self.dX, self.dW = e16(M, N), e16(M, K), e16(N, K)

    def calls(self, i):
        """The two launches of one step: name -> (fn, args, kwargs)."""
        mx, M, N, K, f, m, h = self.mx, self.M, self.N, self.K, self.fmt, self.mode, self.had
        X, W, dY = self.inp[i % len(self.inp)]
        items = [dict(x=X, R=M, C=K, row=self.Xr, col=self.Xc), dict(x=W, R=N, C=K, row=self.Wr, col=self.Wc),
                 dict(x=dY, R=M, C=N, row=self.dYr, col=self.dYc)]
        gemms = [dict(a=self.Xr, b=self.Wr, M=M, N=N, K=K, c=self.Y),      # forward
                 dict(a=self.dYr, b=self.Wc, M=M, N=K, K=N, c=self.dX),    # data gradient
                 dict(a=self.dYc, b=self.Xc, M=N, N=K, K=M, c=self.dW)]    # weight gradient (K = tokens)
        return {"pack_XWdY": (mx.quantize_many, (items, f, m, h), {}),
                "gemm_fwd_dgrad_wgrad": (mx.gemm_many, (gemms, f), {})}

    def run(self, i, T):
        """One step: one launch packs X, W and dY (row + column each), one
        launch computes the forward, data-gradient and weight-gradient
        GEMMs."""
        for n, (fn, a, kw) in self.calls(i).items():
            T.run(n, fn, *a, **kw)

    def flops(self):
        return 3 * 2.0 * self.M * self.N * self.K


def time_steps(fn, steps, warmup, T):
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    T.on = True
    t0 = time.perf_counter()
    for i in range(steps):
        fn(warmup + i)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    T.on = False
    return dt / steps


def capture_steps(step, copies):
    """HIP graphs of whole steps, so that the timed loop replays launches
    without host work in between: graphs[0] holds `copies` consecutive steps
    (input copies 0 .. copies-1, so one replay launches once for that many
    steps), graphs[1 + c] one step on input copy c (for step counts that are
    not a multiple of `copies`).  The captured calls are the same C-ABI
    entry points, enqueued on torch's capture stream."""
    import torch
    T = Timer()
    warm = torch.cuda.Stream()
    warm.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(warm):
        for c in range(copies):
            step.run(c, T)
    torch.cuda.current_stream().wait_stream(warm)
    torch.cuda.synchronize()
    graphs = []
    for group in [list(range(copies))] + [[c] for c in range(copies)]:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for c in group:
                step.run(c, T)
        graphs.append(g)
    torch.cuda.synchronize()
    return graphs


STEP_STATS = {}  # per-replay step times of the last time_graph_steps call


def time_graph_steps(graphs, copies, steps, warmup):
    """Wall time per step of exactly `steps` steps (whole `copies`-step
    graphs, then single-step graphs for the remainder), between two device
    synchronizations, after `warmup` single steps."""
    import torch
    for i in range(warmup):
        graphs[1 + i % copies].replay()
    torch.cuda.synchronize()
    n = steps // copies
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    t0 = time.perf_counter()
    ev[0].record()
    for i in range(n):
        graphs[0].replay()
        ev[i + 1].record()
    for i in range(steps % copies):
        graphs[1 + i].replay()
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / steps
    per = [ev[i].elapsed_time(ev[i + 1]) / copies for i in range(n)]  # ms per step, per replay
    STEP_STATS.clear()
    if per:
        STEP_STATS.update(median_ms=float(np.median(per)), min_ms=float(np.min(per)), replays=n)
    return sec


LAST_GRAPH_TIMES = {}  # statistics of the last graph_time call (us per launch)


def graph_time(launch, reps=10, replays=4, warm=None):
    """Device time of one launch: a graph of `reps` back-to-back calls
    `launch(r)` (r = 0 .. reps-1) replayed `replays` times, a pair of HIP
    events on the replay stream around each replay; the time per call
    excludes host launch cost.  Returns the mean over all replays; the
    median and minimum over replays are left in LAST_GRAPH_TIMES.
    `warm(r)` runs eagerly first (default: `launch`)."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for r in range(reps):
            (warm or launch)(r)
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for r in range(reps):
            launch(r)
    g.replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(replays + 1)]
    ev[0].record()
    for i in range(replays):
        g.replay()
        ev[i + 1].record()
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) * 1e3 / reps for i in range(replays)]
    LAST_GRAPH_TIMES.clear()
    LAST_GRAPH_TIMES.update(mean=float(np.mean(per)), median=float(np.median(per)), min=float(np.min(per)),
                            replays=replays, launches_per_replay=reps)
    return ev[0].elapsed_time(ev[replays]) * 1e3 / (reps * replays)


def sclk_under_load(launch, sample_us=1000, load_ms=6.0):
    """Shader clock (MHz) while `launch(r)` runs back to back: a graph of
    ten launches is replayed for about `load_ms` on the current stream, and
    one wavefront on a second (default-priority) stream counts shader-clock
    cycles against the wall clock for `sample_us` meanwhile (mx_clock_sample).
    That is the clock the kernel actually ran at; random operand data pulls
    it below the 2.4 GHz the datasheet peaks assume."""
    import torch
    from microscaling_block_scaled_mx_amd import mx
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for r in range(10):
            launch(r)
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for r in range(10):
            launch(r)
    g.replay()
    torch.cuda.synchronize()
    ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    ev[0].record()
    g.replay()
    ev[1].record()
    torch.cuda.synchronize()
    reps = max(2, int(load_ms / max(ev[0].elapsed_time(ev[1]), 1e-3)) + 1)
    out = torch.zeros(2, dtype=torch.int64, device="cuda")
    side = torch.cuda.Stream()
    g.replay()  # the load is running before the sample starts
    with torch.cuda.stream(side):
        mx.clock_sample(sample_us, out, stream=side)
    for _ in range(reps - 1):
        g.replay()
    torch.cuda.synchronize()
    cycles, ticks = (int(v) for v in out.cpu())
    khz = mx.wall_clock_khz()
    if ticks <= 0 or khz <= 0:
        return None
    return round(cycles / ticks * khz / 1e3, 1)


KERNEL_STATS = {}  # median / min per launch name from kernel_times


def kernel_times(step):
    """Device time (us) of each of the step's launches, each repeated back to
    back over the rotating input copies."""
    out = {}
    for name in step.calls(0):
        def launch(r, name=name):
            fn, a, kw = step.calls(r)[name]
            fn(*a, **kw)
        out[name] = graph_time(launch, replays=8)
        KERNEL_STATS[name] = dict(LAST_GRAPH_TIMES)
    return out


# ------------------------------------------------------------------ CPU oracle baseline
def cpu_baseline(step: LinearStep, repeats=3):
    """The oracle (never tuned for this) on the host cores, running the whole
    headline step -- dual packs of X, W and dY, then all rows of the fwd,
    dgrad and wgrad GEMMs -- `repeats` times (about 10 s on 16 cores)."""
    from oracle import oracle as orc
    X, W, dY = step.host
    M, N, K, f, m, h = step.M, step.N, step.K, step.fmt, step.mode, step.had
    t0 = time.perf_counter()
    for _ in range(repeats):
        px = orc.quantize(X, M, K, f, m, h, row=True, col=True)
        pw = orc.quantize(W, N, K, f, m, h, row=True, col=True)
        pd = orc.quantize(dY, M, N, f, m, h, row=True, col=True)
        # (A operand, B operand, M, N, K) of the fwd, dgrad and wgrad GEMMs
        for pa, sa, pb, sb, MM, NN, KK in ((px, "row", pw, "row", M, N, K), (pd, "row", pw, "col", M, K, N),
                                           (pd, "col", px, "col", N, K, M)):
            orc.gemm(pa[sa + "_codes"], pa[sa + "_scales"], pb[sb + "_codes"], pb[sb + "_scales"], MM, NN, KK, f)
    total = time.perf_counter() - t0
    cores = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
    return {"value": step.flops() * repeats / total / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{repeats} whole steps (dual packs of X, W, dY + all rows of the fwd, dgrad and wgrad "
                      f"GEMMs), {total / repeats:.2f} s per step",
            "seconds_measured": round(total, 2)}


def cpu_baseline_per_config():
    """The oracle on bounded samples of the other workloads (part of the
    CPU-baseline leg): per workload, one pack on a row slice of its largest
    input (algorithmic bytes / s) and its largest GEMM on a 512-row sample
    of A against all of B (TFLOP/s; the oracle dequantizes B once per call,
    which the rate includes).  About 20 s in all on 16 cores."""
    from microscaling_block_scaled_mx_amd import inputs as I
    from oracle import oracle as orc
    out = {}

    def timed(fn):
        t0 = time.perf_counter()
        r = fn()
        return r, time.perf_counter() - t0

    def sample(name, x, rows, C, fmt, mode, had, pro, aux, B, N, K, extra_in, what):
        xs = np.ascontiguousarray(x[:rows])
        auxs = None if aux is None else np.ascontiguousarray(aux[:rows])
        _, tp = timed(lambda: orc.quantize(xs, rows, C, fmt, mode, had, pro=pro, aux=auxs, row=True, col=True))
        bits = {orc.E2M1: 4, orc.E2M3: 6, orc.E4M3: 8}[fmt]
        pack_bytes = rows * C * (2 + 2 * extra_in + 2 * (bits / 8 + 1 / 32))
        qa = orc.quantize(I.bf16_normal(np.random.default_rng(5), (512, K)), 512, K, fmt, mode, had)
        qb = orc.quantize(B, N, K, fmt, mode, had)
        _, tg = timed(lambda: orc.gemm(qa["row_codes"], qa["row_scales"], qb["row_codes"], qb["row_scales"], 512, N,
                                       K, fmt))
        out[name] = {"pack_gbs": round(pack_bytes / tp / 1e9, 3), "gemm_tflops": round(2.0 * 512 * N * K / tg / 1e12, 4),
                     "sample": what, "seconds": round(tp + tg, 2)}

    A, Bm = I.gemm_pair(101, 256, 256, 256)
    _, t1 = timed(lambda: orc.gemm(*(lambda a, b: (a["row_codes"], a["row_scales"], b["row_codes"], b["row_scales"]))(
        orc.quantize(A, 256, 256, orc.E2M1, orc.FLOOR), orc.quantize(Bm, 256, 256, orc.E2M1, orc.FLOOR)),
        256, 256, 256, orc.E2M1))
    out["mxfp4_256"] = {"us_per_step": round(t1 * 1e6, 1), "sample": "the whole step (packs of A, B and the GEMM)"}
    M, D, F = 8192, 3072, 12288
    X, W1, b1, W2, dY = I.mlp(301, M, D, F)
    # da and h of the backward's dGELU pack (the step computes them; here N(0,1) stand-ins of their shape)
    h = I.bf16_normal(np.random.default_rng(3), (1024, F))
    da = I.bf16_normal(np.random.default_rng(4), (1024, F))
    sample("fused_mlp_mxfp6", da, 1024, F, orc.E2M3, orc.FLOOR, True, orc.PRO_DGELU, h, W1, F, D, 1,
           "dGELU dual pack of (da, h) rows 0-1023 of [8192, 12288]; fc1 GEMM on 512 rows of A (512 x 12288 x 3072)")
    name, K, N = I.FLUX_LINEARS[0]
    Xq, Wq, _ = I.linear(401, 1024, N, K)
    sample("mxfp4_flux_sweep", Xq, 1024, K, orc.E2M1, orc.FLOOR, False, orc.PRO_IDENTITY, None, Wq, N, K, 0,
           "QKV: dual pack of X rows 0-1023 of [16384, 3072]; fwd GEMM on 512 rows of X (512 x 9216 x 3072)")
    counts, offsets, Xg, W1g, W2g, dYg = I.grouped_mlp(501, 32768, 2048, 768, 8)
    sample("grouped_mxfp8", Xg, 1024, 2048, orc.E4M3, orc.RCEIL, False, orc.PRO_IDENTITY, None,
           np.ascontiguousarray(W1g[0]), 1536, 2048, 0,
           "dual pack of X rows 0-1023 of [32768, 2048]; FC1 GEMM of expert 0 on 512 rows (512 x 1536 x 2048)")
    return out


# ------------------------------------------------------------------ other workloads
def bench_linear256(mx, T, iters=20):
    """The 256^3 MXFP4 case: packs of A and B (one launch) and the GEMM with an
    fp32 C.  Device time per step from graph replays (a latency-bound case:
    one 256x256 tile, reported in microseconds)."""
    import torch
    from microscaling_block_scaled_mx_amd import inputs as I
    A, B = I.gemm_pair(101, 256, 256, 256)
    Ad, Bd = dev(A), dev(B)
    pa, pb = mx.alloc_packed(256, 256, mx.E2M1), mx.alloc_packed(256, 256, mx.E2M1)
    C = torch.empty((256, 256), dtype=torch.float32, device="cuda")
    items = [dict(x=Ad, R=256, C=256, row=pa), dict(x=Bd, R=256, C=256, row=pb)]

    def pack(r):
        mx.quantize_many(items, mx.E2M1, mx.FLOOR)

    def gemm(r):
        mx.gemm(pa, pb, 256, 256, 256, mx.E2M1, C, c_dtype=mx.F32)

    def step(r):
        pack(r)
        gemm(r)
    return {"workload": "MXFP4 quantize + GEMM 256^3, fp32 C", "us_per_step": graph_time(step, replays=8),
            "step_median_us": LAST_GRAPH_TIMES["median"], "pack_us": graph_time(pack, replays=8),
            "gemm_us": graph_time(gemm, replays=8)}


def bench_fused_mlp(mx, T, iters=5):
    """Fused MXFP6 MLP (M = 8192, 3072 -> 12288 -> 3072): forward + backward per step, timed as
    replays of a HIP graph of two steps over two copies of the inputs (X,
    W1, b1, W2, dY: 250 MB per copy, so a step does not find its inputs in
    the 256 MB Infinity Cache), after warm-up steps."""
    import torch
    from microscaling_block_scaled_mx_amd import inputs as I
    M, D, F = 8192, 3072, 12288
    X, W1, b1, W2, dY = I.mlp(301, M, D, F)
    P = lambda r, k: mx.alloc_packed(r, k, mx.E2M3)
    e16 = lambda *s: torch.empty(s, dtype=torch.int16, device="cuda")
    ins = [dict(X=dev(X), W1=dev(W1), b1=dev(b1), W2=dev(W2), dY=dev(dY)) for _ in range(2)]
    t = dict(h=e16(M, F), Y=e16(M, D), Xr=P(M, D),
             Xc=P(D, M), W1r=P(F, D), W1c=P(D, F), W2r=P(D, F), W2c=P(F, D), ar=P(M, F), ac=P(F, M),
             da=e16(M, F), dX=e16(M, D), dW1=e16(F, D), dW2=e16(D, F),
             db1=torch.empty(F, dtype=torch.float32, device="cuda"),
             part=torch.empty((M // 32, F), dtype=torch.float32, device="cuda"), dYr=P(M, D), dYc=P(D, M),
             dhr=P(M, F), dhc=P(F, M))

    def fwd(c):
        i = ins[c % 2]
        mx.fused_mlp_fwd(M, D, F, i["X"], i["W1"], i["b1"], i["W2"], t["h"], t["Y"], t["Xr"], t["Xc"], t["W1r"],
                         t["W1c"], t["W2r"], t["W2c"], t["ar"], t["ac"])

    def bwd(c):
        i = ins[c % 2]
        mx.fused_mlp_bwd(M, D, F, i["dY"], t["h"], t["Xc"], t["W1c"], t["W2c"], t["ac"], t["da"], t["dX"], t["dW1"],
                         t["dW2"], t["db1"], t["part"], t["dYr"], t["dYc"], t["dhr"], t["dhc"])

    def step(c):
        fwd(c)
        bwd(c)
    per_step = graph_time(step, reps=2, replays=iters)
    fwd_us = graph_time(fwd, reps=2, replays=iters)
    bwd_us = graph_time(bwd, reps=2, replays=iters)
    fl = 6 * 2.0 * M * D * F
    # the step's floor: its six GEMMs at the MXFP6 peak plus its packs'
    # algorithmic bytes at HBM speed (dual packs of X, W1, W2, dY; the GELU
    # pack of a from h; the dGELU pack of dh from da and h with its 32-row
    # partials; the column-sum finish reading the partials)
    dual = 2 + 2 * PACK_OUT[6]
    pack_bytes = (dual * (M * D + F * D + D * F + M * D) + dual * M * F + (dual + 2 + 0.125) * M * F
                  + 0.125 * M * F)
    floor_us = fl / (PEAK_TFLOPS["fp6"] * 1e6) + pack_bytes / (HBM_GBS * 1e3)
    return {"workload": "fused MXFP6 MLP M=8192 3072->12288->3072 tanh-GELU fwd+bwd (+db1)",
            "launch": "hip_graph (2 steps over 2 input copies per replay)",
            "ms_per_step": per_step / 1e3, "fwd_ms": fwd_us / 1e3, "bwd_ms": bwd_us / 1e3,
            "tflops": fl / (per_step * 1e-6) / 1e12, "frac_of_fp6_peak": fl / (per_step * 1e-6) / 1e12 / PEAK_TFLOPS["fp6"],
            "floor_ms": {"gemms_at_peak": fl / (PEAK_TFLOPS["fp6"] * 1e6) / 1e3,
                         "packs_at_hbm": pack_bytes / (HBM_GBS * 1e3) / 1e3, "total": floor_us / 1e3},
            "frac_of_floor": floor_us / per_step}


def bench_flux_sweep(mx, T, iters=3):
    import torch
    from microscaling_block_scaled_mx_amd import inputs as I
    out = {"workload": "MXFP4 Flux-12B block linears at M=16384, fwd+dgrad+wgrad", "linears": {}}
    tot_fl = tot_gemm_us = tot_us = 0.0
    for i, (name, K, N) in enumerate(I.FLUX_LINEARS):
        # one input set (X, W, dY) under 256 MB would stay in the Infinity
        # Cache across back-to-back launches: rotate two copies of it then
        copies = 2 if 2 * (16384 * K + N * K + 16384 * N) < 256e6 else 1
        st = LinearStep(mx, 16384, N, K, mx.E2M1, mx.FLOOR, False, 401 + i, copies=copies)
        k = kernel_times(st)  # device time of the step's two launches
        g = k["gemm_fwd_dgrad_wgrad"]
        step_us = g + k["pack_XWdY"]
        fl = st.flops()
        out["linears"][name] = {"K": K, "N": N, "gemm_us": g, "step_us": step_us,
                                "gemm_tflops": fl / (g * 1e-6) / 1e12}
        tot_fl += fl
        tot_gemm_us += g
        tot_us += step_us
        del st
        torch.cuda.empty_cache()
    out["gemm_tflops"] = tot_fl / (tot_gemm_us * 1e-6) / 1e12
    out["frac_of_fp4_peak"] = out["gemm_tflops"] / PEAK_TFLOPS["fp4"]
    out["step_tflops"] = tot_fl / (tot_us * 1e-6) / 1e12
    return out


def grouped_buffers(mx, R, D, F, G, X, W1, W2, dY, offsets, fmt):
    """Device inputs, packed operands and outputs of the grouped MLP step."""
    import torch
    P = lambda r, k, b=None: mx.alloc_packed(r, k, fmt, batch=b)
    e16 = lambda *s: torch.empty(s, dtype=torch.int16, device="cuda")
    return dict(X=dev(X), W1=dev(W1), W2=dev(W2), dY=dev(dY), off=dev(offsets.astype(np.int32)), Xr=P(R, D),
                Xc=P(D, R), W1r=P(2 * F, D, G), W1c=P(D, 2 * F, G), W2r=P(D, F, G), W2c=P(F, D, G), H=e16(R, 2 * F),
                zr=P(R, F), zc=P(F, R), Y=e16(R, D), dYr=P(R, D), dYc=P(D, R), dHr=P(R, 2 * F), dHc=P(2 * F, R),
                dX=e16(R, D), dW1=e16(G, 2 * F, D), dW2=e16(G, D, F))


_STEP_EVENTS = {}  # the two-stream schedule's events, made once per side stream


def grouped_step(mx, t, R, D, F, G, fmt, mode, T=None, side=None):
    """One grouped SwiGLU MLP step (forward + backward) through the C ABI.

    side=None: every launch in order on the current stream (each timed by T
    when given).  side=<stream>: the same launches, those that do not depend
    on each other on two streams -- the weight and dY packs beside the X pack
    and the forward, and each ragged-K weight gradient beside the data
    gradient issued after it, so that its tiles fill the compute units the
    other leaves idle in its last round.  No two concurrent launches write
    the same buffer, so the results are the one-stream schedule's."""
    import torch
    run = (lambda name, fn, *a, **kw: T.run(name, fn, *a, **kw)) if T is not None else \
        (lambda name, fn, *a, **kw: fn(*a, **kw))
    pack_w1 = lambda: run("pack", mx.quantize, t["W1"], 2 * F, D, fmt, mode, row=t["W1r"], col=t["W1c"], batch=G)
    pack_w2 = lambda: run("pack", mx.quantize, t["W2"], D, F, fmt, mode, row=t["W2r"], col=t["W2c"], batch=G)
    pack_x = lambda: run("pack", mx.quantize, t["X"], R, D, fmt, mode, row=t["Xr"], col=t["Xc"])
    pack_dy = lambda: run("pack", mx.quantize, t["dY"], R, D, fmt, mode, row=t["dYr"], col=t["dYc"])
    fc1 = lambda: run("fc1_swiglu", mx.grouped_gemm, mx.RAGGED_M, G, R, t["off"], t["Xr"], t["W1r"], t["H"],
                      epilogue=mx.EPI_SWIGLU, N=2 * F, K=D, out_row=t["zr"], out_col=t["zc"], fmt=fmt,
                      scale_mode=mode)
    fc2 = lambda: run("fc2", mx.grouped_gemm, mx.RAGGED_M, G, R, t["off"], t["zr"], t["W2r"], t["Y"], N=D, K=F,
                      fmt=fmt, scale_mode=mode)
    fc2_dgrad = lambda: run("fc2_dgrad_dswiglu", mx.grouped_gemm, mx.RAGGED_M, G, R, t["off"], t["dYr"],
                            t["W2c"], None, epilogue=mx.EPI_DSWIGLU, N=F, K=D, aux=t["H"], out_row=t["dHr"],
                            out_col=t["dHc"], fmt=fmt, scale_mode=mode)
    fc1_dgrad = lambda: run("fc1_dgrad", mx.grouped_gemm, mx.RAGGED_M, G, R, t["off"], t["dHr"], t["W1c"],
                            t["dX"], N=D, K=2 * F, fmt=fmt, scale_mode=mode)
    wgrad2 = lambda: run("wgrad2", mx.grouped_gemm, mx.RAGGED_K, G, R, t["off"], t["dYc"], t["zc"], t["dW2"],
                         M=D, N=F, fmt=fmt, scale_mode=mode)
    wgrad1 = lambda: run("wgrad1", mx.grouped_gemm, mx.RAGGED_K, G, R, t["off"], t["dHc"], t["Xc"], t["dW1"],
                         M=2 * F, N=D, fmt=fmt, scale_mode=mode)
    if side is None:
        for f in (pack_x, pack_w1, pack_w2, fc1, fc2, pack_dy, fc2_dgrad, fc1_dgrad, wgrad2, wgrad1):
            f()
        return
    main = torch.cuda.current_stream()
    ev = _STEP_EVENTS.setdefault(id(side), [torch.cuda.Event() for _ in range(4)])
    side.wait_stream(main)
    with torch.cuda.stream(side):
        pack_w1()
        pack_w2()
        ev[0].record(side)
        pack_dy()
        ev[1].record(side)
    pack_x()
    main.wait_event(ev[0])
    fc1()
    ev[2].record(main)
    fc2()
    main.wait_event(ev[1])
    with torch.cuda.stream(side):
        side.wait_event(ev[2])
        wgrad2()
    fc2_dgrad()
    ev[3].record(main)
    with torch.cuda.stream(side):
        side.wait_event(ev[3])
        wgrad1()
    fc1_dgrad()
    main.wait_stream(side)


def bench_grouped_mlp(mx, T, iters=5):
    import torch
    from microscaling_block_scaled_mx_amd import inputs as I
    R, D, F, G = 32768, 2048, 768, 8
    counts, offsets, X, W1, W2, dY = I.grouped_mlp(501, R, D, F, G)
    fmt, mode = mx.E4M3, mx.RCEIL
    t = grouped_buffers(mx, R, D, F, G, X, W1, W2, dY, offsets, fmt)
    side = torch.cuda.Stream()  # default priority, like the main stream
    sec_serial = time_steps(lambda i: grouped_step(mx, t, R, D, F, G, fmt, mode, T=T), iters, 2, T)
    k = T.summary()
    sec = time_steps(lambda i: grouped_step(mx, t, R, D, F, G, fmt, mode, side=side), iters, 2, Timer())
    fl = 2.0 * R * D * F * (2 + 1 + 1 + 2 + 1 + 2)
    gemm_us = sum(v for n, v in k.items() if n != "pack")
    out = {"workload": "MXFP8 grouped SwiGLU MLP G=8 D=2048 F=768 R=32768 (one empty expert), fwd+bwd",
           "counts": [int(c) for c in counts], "ms_per_step": sec * 1e3, "step_tflops": fl / sec / 1e12,
           "schedule": "two streams: weight / dY packs and the ragged-K weight gradients beside the main chain",
           "ms_per_step_one_stream": sec_serial * 1e3,
           "gemm_tflops": fl / (gemm_us * 1e-6) / 1e12, "kernels_us": k}
    out["frac_of_fp8_peak"] = out["gemm_tflops"] / PEAK_TFLOPS["fp8"]
    # the step's floor: its GEMMs at the MXFP8 peak plus the standalone dual
    # packs' algorithmic bytes (X, W1, W2, dY) at HBM speed (the epilogues'
    # bytes move inside the GEMM launches)
    pack_bytes = (2 + 2 * PACK_OUT[8]) * (R * D + G * 2 * F * D + G * D * F + R * D)
    floor_us = fl / (PEAK_TFLOPS["fp8"] * 1e6) + pack_bytes / (HBM_GBS * 1e3)
    out["floor_ms"] = {"gemms_at_peak": fl / (PEAK_TFLOPS["fp8"] * 1e6) / 1e3,
                       "packs_at_hbm": pack_bytes / (HBM_GBS * 1e3) / 1e3, "total": floor_us / 1e3}
    out["frac_of_floor"] = floor_us / (sec * 1e6)
    return out


def bench_main_grad(mx, T):
    """The headline weight gradient (MXFP6, dW [3072,3072] = dY^T X over
    4096 tokens) stored into a bf16 main_grad (mx_gemm, beta = 0) and added
    into it (mx_gemm_accumulate, beta = 1), device time per launch."""
    import torch
    M, N, K = 4096, 3072, 3072
    g = torch.Generator(device="cuda").manual_seed(9)
    P = lambda r, k: tuple(torch.randint(118 if i else 0, 130 if i else 256, t.shape, dtype=torch.uint8,
                                         device="cuda", generator=g)
                           for i, t in enumerate(mx.alloc_packed(r, k, mx.E2M3)))
    dyc, xc = P(N, M), P(K, M)
    main_grad = torch.zeros((N, K), dtype=torch.int16, device="cuda")
    fl = 2.0 * M * N * K
    store = graph_time(lambda r: mx.gemm(dyc, xc, N, K, M, mx.E2M3, main_grad))
    accum = graph_time(lambda r: mx.gemm_accumulate(dyc, xc, N, K, M, mx.E2M3, main_grad))
    return {"workload": "MXFP6 wgrad dW[3072,3072] (K = 4096 tokens) into a bf16 main_grad",
            "store_us": store, "accumulate_us": accum, "store_tflops": fl / (store * 1e-6) / 1e12,
            "accumulate_tflops": fl / (accum * 1e-6) / 1e12}


def bench_sr_pack(mx, T):
    """MXFP4 gradient pack (dY of the out-projection at M = 16384, [16384,
    3072], row + column) with stochastic rounding against nearest rounding,
    device time per launch."""
    from microscaling_block_scaled_mx_amd import inputs as I
    R, C = 16384, 3072
    x = dev(I.bf16_normal(np.random.default_rng(11), (R, C)))
    row, col = mx.alloc_packed(R, C, mx.E2M1), mx.alloc_packed(C, R, mx.E2M1)
    rn = graph_time(lambda r: mx.quantize(x, R, C, mx.E2M1, mx.FLOOR, row=row, col=col))
    sr = graph_time(lambda r: mx.quantize_sr(x, R, C, 1234 + r, row=row, col=col))
    b = R * C * (2 + 2 * PACK_OUT[4])
    return {"workload": "MXFP4 dual pack of dY [16384,3072]: stochastic vs nearest rounding",
            "nearest_us": rn, "sr_us": sr, "nearest_gbs": b / (rn * 1e-6) / 1e9, "sr_gbs": b / (sr * 1e-6) / 1e9}


# the dense tilings mx_gemm_tiled serves: (tile_m, tile_n, workgroups per CU)
DENSE_TILES = ((256, 256, 1), (256, 192, 1), (192, 256, 1), (192, 192, 1), (256, 128, 1), (256, 128, 2),
               (128, 256, 2), (192, 192, 2))
SPLITS = (1, 2, 3, 4, 6, 8, 12, 16)
# Flux-12B (hidden 3072) block linears: name -> (N, K) of the forward GEMM
FLUX_LINEARS = {"qkv": (9216, 3072), "out": (3072, 3072), "mlp_up": (12288, 3072), "mlp_down": (3072, 12288),
                "adaln": (18432, 3072)}


def random_packed(mx, rows, K, fmt, gen):
    """A packed operand of random code bytes and E8M0 scales near 2^0."""
    import torch
    codes, scales = mx.alloc_packed(rows, K, fmt)
    codes.copy_(torch.randint(0, 256, codes.shape, dtype=torch.uint8, device="cuda", generator=gen))
    scales.copy_(torch.randint(118, 130, scales.shape, dtype=torch.uint8, device="cuda", generator=gen))
    return codes, scales


def sustained_time(launch, target_ms=6.0, warm_replays=2, replays=4):
    """Device time per call of launch() under sustained load: a graph of as
    many back-to-back calls as fill about target_ms, replayed warm_replays
    times untimed (the clock settles under the kernel's own power draw),
    then replays times between events.  Short bursts run at a higher clock
    than sustained work, so plans are compared this way."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        launch()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        launch()
        e1.record()
    s.synchronize()
    est_us = max(e0.elapsed_time(e1) * 1e3, 1.0)
    reps = int(min(max(target_ms * 1e3 / est_us, 4), 2000))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            launch()
    for _ in range(warm_replays):
        g.replay()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(replays):
        g.replay()
    ev[1].record()
    torch.cuda.synchronize()
    return ev[0].elapsed_time(ev[1]) * 1e3 / (reps * replays)


def time_plan(mx, pa, pb, M, N, K, fmt, C, tile, split, ws):
    return sustained_time(lambda: mx.gemm_splitk(pa, pb, M, N, K, fmt, C, tile, split, ws if split > 1 else None))


def rule_tile(M, N, cus):
    """mx_gemm's rule without the tuned table: of the one-per-CU tilings
    that divide M x N, the fewest rounds x tile area, the first on ties."""
    best, cost = None, None
    for tile in DENSE_TILES:
        if tile[2] != 1 or M % tile[0] or N % tile[1]:
            continue
        tiles = (M // tile[0]) * (N // tile[1])
        c = -(-tiles // cus) * tile[0] * tile[1]
        if cost is None or c < cost:
            best, cost = tile, c
    return best


def tune_shape(mx, M, N, K, fmt, gen, cus=256):
    """Every dense tiling and K split of one GEMM shape, timed under
    sustained load; returns the rule's plan and time (the mean of one timing
    before and one after the candidates) and the best plan and time.  K
    splits are tried only where the tiling has fewer than two rounds of
    tiles.  A best plan more than 5% ahead is re-timed against the rule in
    the order plan, rule, rule, plan, twice; the means of those decide."""
    import torch
    pa, pb = random_packed(mx, M, K, fmt, gen), random_packed(mx, N, K, fmt, gen)
    C = torch.empty((M, N), dtype=torch.int16, device="cuda")
    cands = []
    for tile in DENSE_TILES:
        if M % tile[0] or N % tile[1]:
            continue
        tiles = (M // tile[0]) * (N // tile[1])
        for split in SPLITS:
            if K % (128 * split) or (split > 1 and tiles * tile[2] >= 2 * cus):
                continue
            cands.append((tile, split))
    ws_elems = max(sp * M * N for _, sp in cands)
    ws = torch.empty((ws_elems,), dtype=torch.float32, device="cuda") if ws_elems > M * N else None
    rt = rule_tile(M, N, cus)
    t = lambda tile, split: time_plan(mx, pa, pb, M, N, K, fmt, C, tile, split, ws)
    rule0 = t(rt, 1)
    times = {c: t(*c) for c in cands}
    rule = 0.5 * (rule0 + t(rt, 1))
    best = min(times, key=times.get)
    r = {"M": M, "N": N, "K": K, "fmt": fmt, "rule": list(rt), "rule_us": rule, "best": [list(best[0]), best[1]],
         "best_us": times[best], "candidates": len(cands)}
    if times[best] < 0.95 * rule and best != (rt, 1):
        seq = [t(*best), t(rt, 1), t(rt, 1), t(*best), t(*best), t(rt, 1), t(rt, 1), t(*best)]
        r["confirm_best_us"] = float(np.mean([seq[0], seq[3], seq[4], seq[7]]))
        r["confirm_rule_us"] = float(np.mean([seq[1], seq[2], seq[5], seq[6]]))
    del pa, pb, C, ws
    return r


def tune_gemms(mx, fmts, tokens):
    """The tuned-table sweep: the fwd, dgrad and wgrad GEMMs of every
    Flux-12B block linear at each token count, in each format.  Prints one
    JSON line per shape and, for those whose best plan beat the rule by more
    than 5% in the confirming re-timings, the initializer line of the tuned
    table."""
    import torch
    gen = torch.Generator(device="cuda").manual_seed(11)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    shapes = []
    for T in tokens:
        for name, (N, K) in FLUX_LINEARS.items():
            for M_, N_, K_ in ((T, N, K), (T, K, N), (N, K, T)):
                if (M_, N_, K_) not in shapes:
                    shapes.append((M_, N_, K_))
    lines = []
    for fmt in fmts:
        for M, N, K in shapes:
            r = tune_shape(mx, M, N, K, fmt, gen, cus)
            print(json.dumps({"tune": r}), flush=True)
            if "confirm_best_us" in r and r["confirm_best_us"] < 0.95 * r["confirm_rule_us"]:
                (tm, tn, wg), sp = r["best"]
                lines.append(f"    {{{cus}, {fmt}, {M}, {N}, {K}, {{{tm}, {tn}, {wg}, {sp}}}}},  "
                             f"// {r['confirm_rule_us']:.1f} -> {r['confirm_best_us']:.1f} us")
            torch.cuda.empty_cache()
    for ln in lines:
        print(ln, flush=True)


def bench_tuned_plans(mx, T):
    """The tuned table's split-K plans against mx_gemm's rule: the dgrad
    GEMMs of the Flux-12B QKV, MLP and adaLN linears at 512 tokens (few
    output tiles, long K) in each format, random code bytes.  Each time is
    under sustained load (see sustained_time), taken in the order plan,
    rule, rule, plan; the planned call includes its reduction."""
    import torch
    gen = torch.Generator(device="cuda").manual_seed(13)
    out = {"workload": "dgrad GEMMs of the Flux-12B QKV / MLP / adaLN linears at 512 tokens (M=512, N=3072, "
                       "K=9216/12288/18432): mx_gemm (rule) vs mx_gemm_splitk under mx_gemm_plan", "shapes": {}}
    for fbits, fmt in (("4", mx.E2M1), ("6", mx.E2M3), ("8", mx.E4M3)):
        for K in (9216, 12288, 18432):
            M, N = 512, 3072
            pa, pb = random_packed(mx, M, K, fmt, gen), random_packed(mx, N, K, fmt, gen)
            C = torch.empty((M, N), dtype=torch.int16, device="cuda")
            tile, split, wsb = mx.gemm_plan(M, N, K, fmt)
            ws = torch.empty((max(wsb // 4, 1),), dtype=torch.float32, device="cuda")
            f_rule = lambda: mx.gemm(pa, pb, M, N, K, fmt, C)
            f_plan = lambda: mx.gemm_planned(pa, pb, M, N, K, fmt, C, workspace=ws)
            seq = [sustained_time(f) for f in (f_plan, f_rule, f_rule, f_plan)]
            rule, plan = 0.5 * (seq[1] + seq[2]), 0.5 * (seq[0] + seq[3])
            fl = 2.0 * M * N * K
            out["shapes"][f"mxfp{fbits}_{M}x{N}x{K}"] = {
                "plan": {"tile": list(tile), "split_k": split}, "rule_us": round(rule, 2), "plan_us": round(plan, 2),
                "speedup": round(rule / plan, 3), "plan_tflops": round(fl / (plan * 1e-6) / 1e12, 1)}
            del pa, pb, C, ws
    return out


def only(mx, spec, steps, warmup, T):
    """One kernel configuration, for profilers: gemm:FMT:M:N:K, pack:FMT:R:C
    (dual pack), packs:FMT:M:N:K (the linear step's fused dual packs of X,
    W and dY), gemms:FMT:M:N:K (its three GEMMs in one launch; random
    codes) or copy:BYTES; or one whole other workload: linear256, mlp,
    sweep, grouped, main_grad, sr_pack or tuned.  Prints one JSON line with
    its average time."""
    import torch
    from microscaling_block_scaled_mx_amd import inputs as I
    workloads = {"linear256": bench_linear256, "mlp": bench_fused_mlp, "sweep": bench_flux_sweep, "grouped": bench_grouped_mlp,
                 "main_grad": bench_main_grad, "sr_pack": bench_sr_pack, "tuned": bench_tuned_plans}
    if spec in workloads:  # one of the other workloads, as in the full run
        print(json.dumps({"only": spec, **workloads[spec](mx, T)}), flush=True)
        return
    kind, fbits, *dims = spec.split(":")
    if kind == "tune":  # tune:FMTS:TOKENS, e.g. tune:4,6,8:512,1024 -- the tuned-table sweep
        fmts = [{"4": mx.E2M1, "6": mx.E2M3, "8": mx.E4M3}[f] for f in fbits.split(",")]
        tune_gemms(mx, fmts, [int(t) for t in dims[0].split(",")] if dims else [512, 1024, 2048, 4096, 8192,
                                                                                16384])
        return
    if kind == "copy":  # plain device copy of fbits bytes: the reference for the traffic counters
        n = int(fbits)
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        us = graph_time(lambda r: dst.copy_(src), reps=steps)
        print(json.dumps({"only": spec, "us": us, "gbs": 2 * n / (us * 1e-6) / 1e9}), flush=True)
        return
    fmt = {"4": mx.E2M1, "6": mx.E2M3, "8": mx.E4M3}[fbits]
    mode = mx.RCEIL if fmt == mx.E4M3 else mx.FLOOR
    had = fmt == mx.E2M3
    if kind == "gemm":
        M, N, K = (int(v) for v in dims)
        A, B = I.gemm_pair(7, M, N, K, 1.0, 0.02)
        pa, pb = mx.alloc_packed(M, K, fmt), mx.alloc_packed(N, K, fmt)
        mx.quantize(dev(A), M, K, fmt, mode, had, row=pa)
        mx.quantize(dev(B), N, K, fmt, mode, had, row=pb)
        C = torch.empty((M, N), dtype=torch.int16, device="cuda")
        us = graph_time(lambda r: mx.gemm(pa, pb, M, N, K, fmt, C), reps=steps)
        print(json.dumps({"only": spec, "us": us, "tflops": 2.0 * M * N * K / (us * 1e-6) / 1e12}), flush=True)
    elif kind == "gemmk":  # one GEMM with a forced tiling and K split: FMT:M:N:K:BM:BN:WG_PER_CU:SPLIT
        M, N, K, bm, bn, occ, split = (int(v) for v in dims[:7])
        g = torch.Generator(device="cuda").manual_seed(7)
        pa, pb = random_packed(mx, M, K, fmt, g), random_packed(mx, N, K, fmt, g)
        C = torch.empty((M, N), dtype=torch.int16, device="cuda")
        ws = torch.empty((split * M * N,), dtype=torch.float32, device="cuda") if split > 1 else None
        us = time_plan(mx, pa, pb, M, N, K, fmt, C, (bm, bn, occ), split, ws)
        print(json.dumps({"only": spec, "us": us, "tflops": 2.0 * M * N * K / (us * 1e-6) / 1e12}), flush=True)
    elif kind == "gemmt":  # one GEMM with a forced tiling: FMT:M:N:K:BM:BN:WG_PER_CU[:rand|zero]
        M, N, K, bm, bn, occ = (int(v) for v in dims[:6])
        data = dims[6] if len(dims) > 6 else "rand"
        g = torch.Generator(device="cuda").manual_seed(7)

        def fill(i, t):
            if i:
                return torch.randint(118, 130, t.shape, dtype=torch.uint8, device="cuda", generator=g)
            if data == "zero":
                return torch.zeros_like(t)
            return torch.randint(0, 256, t.shape, dtype=torch.uint8, device="cuda", generator=g)
        pa, pb = (tuple(fill(i, t) for i, t in enumerate(mx.alloc_packed(r, K, fmt))) for r in (M, N))
        C = torch.empty((M, N), dtype=torch.int16, device="cuda")
        us = graph_time(lambda r: mx.gemm_tiled(pa, pb, M, N, K, fmt, C, (bm, bn, occ)), reps=steps)
        print(json.dumps({"only": spec, "data": data, "us": us, "tflops": 2.0 * M * N * K / (us * 1e-6) / 1e12}),
              flush=True)
    elif kind == "gemms":  # the linear step's three GEMMs in one launch (FMT:M:N:K as the step)
        # optional 5th field: operand data -- rand (random code bytes, the
        # default), zero (all codes +0) or const (one non-zero code byte
        # everywhere): the matrix cores' clock under load depends on how
        # many operand bits toggle, so the three bound what data costs
        M, N, K = (int(v) for v in dims[:3])
        data = dims[3] if len(dims) > 3 else "rand"
        g = torch.Generator(device="cuda").manual_seed(7)

        def fill(i, t):
            if i:  # scales: E8M0 bytes near 2^0
                return torch.randint(118, 130, t.shape, dtype=torch.uint8, device="cuda", generator=g)
            if data == "zero":
                return torch.zeros_like(t)
            if data == "const":
                return torch.full_like(t, 0x5A)
            return torch.randint(0, 256, t.shape, dtype=torch.uint8, device="cuda", generator=g)
        P = lambda r, k: tuple(fill(i, t) for i, t in enumerate(mx.alloc_packed(r, k, fmt)))
        trio = [(P(M, K), P(N, K), M, N, K), (P(M, N), P(K, N), M, K, N), (P(N, M), P(K, M), N, K, M)]
        items = [dict(a=a, b=b, M=m, N=n, K=k, c=torch.empty((m, n), dtype=torch.int16, device="cuda"))
                 for a, b, m, n, k in trio]
        us = graph_time(lambda r: mx.gemm_many(items, fmt), reps=steps)
        sclk = sclk_under_load(lambda r: mx.gemm_many(items, fmt))
        print(json.dumps({"only": spec, "data": data, "us": us, "tflops": 3 * 2.0 * M * N * K / (us * 1e-6) / 1e12,
                          "sclk_mhz": sclk}), flush=True)
    elif kind == "packs":  # the linear step's fused pack: X [M,K], W [N,K], dY [M,N] in one launch
        M, N, K = (int(v) for v in dims)
        rng = np.random.default_rng(7)
        shapes = ((M, K), (N, K), (M, N))
        xs = [dev(I.bf16_normal(rng, sh)) for sh in shapes]
        items = [dict(x=x, R=r, C=c, row=mx.alloc_packed(r, c, fmt), col=mx.alloc_packed(c, r, fmt))
                 for x, (r, c) in zip(xs, shapes)]
        us = graph_time(lambda r: mx.quantize_many(items, fmt, mode, had), reps=steps)
        b = sum(r * c for r, c in shapes) * (2 + 2 * PACK_OUT[int(fbits)])
        print(json.dumps({"only": spec, "us": us, "gbs": b / (us * 1e-6) / 1e9}), flush=True)
    else:
        R, C = (int(v) for v in dims)
        X = dev(I.bf16_normal(np.random.default_rng(7), (R, C)))
        row, col = mx.alloc_packed(R, C, fmt), mx.alloc_packed(C, R, fmt)
        us = graph_time(lambda r: mx.quantize(X, R, C, fmt, mode, had, row=row, col=col), reps=steps)
        b = R * C * (2 + 2 * PACK_OUT[int(fbits)])
        print(json.dumps({"only": spec, "us": us, "gbs": b / (us * 1e-6) / 1e9}), flush=True)


# ------------------------------------------------------------------ main
def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)  # ~13 ms timed: fixed host latency < 1% of it
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--extra", choices=["all", "none"], default="all")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead of graph replays")
    ap.add_argument("--only", default=None,
                    help="profile one kernel config instead: gemm:FMT:M:N:K, pack:FMT:R:C, packs:FMT:M:N:K, "
                         "gemms:FMT:M:N:K, gemmt:FMT:M:N:K:BM:BN:WG, gemmk:FMT:M:N:K:BM:BN:WG:SPLIT "
                         "(FMT = 4, 6 or 8), copy:BYTES (a plain device copy), tune:FMTS:TOKENS (the tuned "
                         "GEMM table's sweep), or one workload: "
                         "linear256, mlp, sweep, grouped, main_grad, sr_pack, tuned")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this path has no multi-GPU mode (each GPU would run the same "
              "kernels on its own shard); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from microscaling_block_scaled_mx_amd import mx
    if not torch.cuda.is_available() or not mx.device_supported(0):
        print("bench.py needs a gfx950 GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    T = Timer()
    if args.only:
        only(mx, args.only, args.steps, args.warmup, T)
        return
    M, N, K = 4096, 3072, 3072
    step = LinearStep(mx, M, N, K, mx.E2M3, mx.FLOOR, True, 201)
    print(f"[bench] linear MXFP6 {M}x{N}x{K}: warmup {args.warmup}, steps {args.steps}", file=sys.stderr,
          flush=True)
    if args.no_graph:
        sec = time_steps(lambda i: step.run(i, T), args.steps, args.warmup, Timer())
    else:
        graphs = capture_steps(step, len(step.inp))
        sec = time_graph_steps(graphs, len(step.inp), args.steps, args.warmup)
    # per-launch device durations (graphs of repeated launches, after the
    # timed steps)
    k = kernel_times(step)
    value = step.flops() / sec / 1e12
    gemm_us = k["gemm_fwd_dgrad_wgrad"]
    gemm_flops = step.flops()  # the three GEMMs of the one launch
    achieved = gemm_flops / (gemm_us * 1e-6) / 1e12
    # algorithmic bytes of the fused pack: X [M,K], W [N,K], dY [M,N], each read once (bf16) and written twice
    pack_bytes = (M * K + N * K + M * N) * (2 + 2 * PACK_OUT[6])
    # the shader clock while each launch runs back to back (mx_clock_sample)
    def call_of(name):
        return lambda r: (lambda fn, a, kw: fn(*a, **kw))(*step.calls(r)[name])
    sclk = {n: sclk_under_load(call_of(n)) for n in ("gemm_fwd_dgrad_wgrad", "pack_XWdY")}
    kernels = {n: {"us": round(v, 2), "median_us": round(KERNEL_STATS[n]["median"], 2),
                   "min_us": round(KERNEL_STATS[n]["min"], 2)} for n, v in k.items()}
    kernels["gemm_fwd_dgrad_wgrad"]["tflops"] = round(achieved, 1)
    kernels["pack_XWdY"]["gbs"] = round(pack_bytes / (k["pack_XWdY"] * 1e-6) / 1e9, 1)
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(sec * 1e3, 4),
        "ms_per_step_median": round(STEP_STATS["median_ms"], 4) if STEP_STATS else None,
        "ms_per_step_min": round(STEP_STATS["min_ms"], 4) if STEP_STATS else None,
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "mxfp6 (e2m3 x e2m3, fp32 accumulate)", "data": "synthetic",
        "launch": "eager" if args.no_graph else "hip_graph (4 consecutive steps per graph)",
        "config": {"workload": "MXFP6 linear (E2M3, FLOOR, Hadamard-32) X[4096,3072] W[3072,3072]: dual packs "
                               "of X, W, dY + fwd, dgrad, wgrad GEMMs, bf16 out",
                   "M": M, "N": N, "K": K, "format": "mxfp6", "gemm_flops_per_step": step.flops()},
        "roofline": {"bound": "mfma", "kernel": "gemm_many_kernel<E2M3, 256x192 | 192x192> (fwd, dgrad and wgrad "
                                                "in one launch, 231.9 GFLOP)",
                     "achieved": round(achieved, 1), "peak": PEAK_TFLOPS["fp6"], "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_TFLOPS["fp6"], 4), "traffic": measured_traffic(GEMM_TRAFFIC),
                     "traffic_unit": "bytes per launch (HBM read + write)",
                     "sclk_mhz": sclk["gemm_fwd_dgrad_wgrad"],
                     "peak_at_sclk": (round(PEAK_TFLOPS["fp6"] * sclk["gemm_fwd_dgrad_wgrad"] / 2400.0, 1)
                                      if sclk["gemm_fwd_dgrad_wgrad"] else None)},
        "quantizer": {"kernel": "pack_many_kernel<E2M3, Hadamard>: dual packs of X, W and dY in one launch",
                      "achieved_gbs": round(pack_bytes / (k["pack_XWdY"] * 1e-6) / 1e9, 1), "peak_gbs": HBM_GBS,
                      "frac": round(pack_bytes / (k["pack_XWdY"] * 1e-6) / 1e9 / HBM_GBS, 4),
                      "algorithmic_bytes": pack_bytes, "traffic": measured_traffic(PACK_TRAFFIC),
                      "alu": alu_roofline(k["pack_XWdY"]), "sclk_mhz": sclk["pack_XWdY"]},
        "kernels": kernels,
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu oracle baseline", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(step)
        if args.extra == "all":
            line["cpu_baseline"]["per_workload"] = cpu_baseline_per_config()
    if args.extra == "all":
        extra = {}
        for name, fn in (("mxfp4_256", bench_linear256), ("fused_mlp_mxfp6", bench_fused_mlp), ("mxfp4_flux_sweep", bench_flux_sweep),
                         ("grouped_mxfp8", bench_grouped_mlp), ("wgrad_main_grad", bench_main_grad),
                         ("mxfp4_sr_pack", bench_sr_pack), ("tuned_splitk_512_tokens", bench_tuned_plans)):
            print(f"[bench] {name}", file=sys.stderr, flush=True)
            extra[name] = fn(mx, T)
            torch.cuda.empty_cache()
        line["extra"] = extra
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
