#!/usr/bin/env python3
"""Benchmark of the staged tensor-parallel GEMM share on one MI355X.

Default workload: the fp8 all-gather GEMM rank share, P = 8: A e4m3
8192 x 8192 in eight ring-ordered 1024-row slices, B e4m3 1024 x 8192 (N x K),
C bf16 8192 x 1024, alpha = beta = 1, bf16 out. One step is one full call of
tpgemm_stage_ag as the library issues it by default: the seven slice
deliveries back to back in ring order, the local stage beside them, the
remote stages gated on their deliveries, the fused alpha/beta epilogue (the
call fans out over streams, so it is issued eagerly; a replayed hipGraph of
it is reported in "detail"). Inputs are resident in HBM before the timed
region starts.

Prints ONE JSON line. Diagnostics (compute-only time, delivery-only time,
hidden fraction, unstaged time, L2-flushed time) go into its "detail" object
and to stderr, together with the rest of the metric, every run: the P = 2
bf16 all-gather, the bf16 reduce-scatter, the SwiGLU block and the per-slot
FFN layer (each with its stage GEMM launches against the bf16 MFMA peak; the
FFN split into its first GEMM, LayerNorm / SiLU pass and second GEMM), and
the dispatch / combine permutes against the HBM peak. --all adds the
backward pass, the column-dual schedules and the fused QKV projection;
--sweep adds the delivered-bytes / compute scale sweep.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline] [--all] [--sweep]
"""
import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import comm_overlapped_linear_amd as tp  # noqa: E402
from synth import workloads as W  # noqa: E402

METRIC = "staged TP-GEMM TFLOP/s + % MFMA peak (bf16/fp8) on 1 GPU; FFN-layer µs"
PEAK_TFLOPS = {"fp8_e4m3": 5000.0, "bf16": 2500.0}     # MI355X dense MFMA peaks
HBM_PEAK_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def dev(bits):
    view = np.int16 if bits.dtype == np.uint16 else np.uint8
    return torch.from_numpy(np.ascontiguousarray(bits).view(view)).cuda()


def time_steps(fn, steps, warmup):
    """ms per call over `steps` calls, after `warmup` calls and at least
    WARM_MS of calls (the clocks settle over the first few ms of load)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < WARM_MS:
        fn()
        torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(steps):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / steps


WARM_MS = 30.0


def time_flushed(fn, steps, warmup, scratch):
    """Per-call times with the caches flushed (a 512 MiB write) before each call."""
    for _ in range(warmup):
        fn()
    times = []
    for _ in range(steps):
        scratch.add_(1)
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        torch.cuda.synchronize()
        times.append(s.elapsed_time(e))
    times = times[1:] if len(times) > 1 else times
    return dict(mean=float(np.mean(times)), min=float(np.min(times)), max=float(np.max(times)),
                median=float(np.median(times)))


def time_sustained(fn, seconds=1.0, batch=50):
    """Throughput of back-to-back calls held for about `seconds` (the clocks
    the chip settles at under sustained load): ms per call over the whole run."""
    fn()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    calls, t0 = 0, time.perf_counter()
    s.record()
    while time.perf_counter() - t0 < seconds:
        for _ in range(batch):
            fn()
        calls += batch
        torch.cuda.synchronize()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / calls, calls


def measure_mfma_peaks():
    """The matrix cores' attainable rate on this chip: a register-only MFMA
    loop over every CU (no memory traffic), timed with events, plus the
    engine clock it ran at (shader-clock over wall-clock ticks)."""
    cus, clk_khz, wall_khz = tp.device_info()
    blocks = 2 * cus                       # 16 waves per CU
    sink = torch.zeros(blocks * 8 * 2, dtype=torch.int64, device="cuda")
    out = dict(cus=cus, spec_clock_mhz=round(clk_khz / 1e3), wall_clock_mhz=round(wall_khz / 1e3, 1))
    for name, dt, iters in (("e4m3", tp.E4M3, 16000), ("bf16", tp.BF16, 32000)):
        tp.mfma_probe(dt, iters // 2, blocks, sink)              # clocks settle
        torch.cuda.synchronize()
        best = None
        for _ in range(3):
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            flop = tp.mfma_probe(dt, iters, blocks, sink)
            e.record()
            torch.cuda.synchronize()
            ms = s.elapsed_time(e)
            if best is None or ms < best[0]:
                ticks = sink.view(-1, 2).cpu().numpy().astype(np.float64)
                best = (ms, flop, float(np.median(ticks[:, 0] / ticks[:, 1])) * wall_khz / 1e3)
        ms, flop, mhz = best
        spec = PEAK_TFLOPS["fp8_e4m3" if name == "e4m3" else "bf16"]
        tf = flop / (ms * 1e-3) / 1e12
        out[name] = dict(tflops=round(tf, 1), frac_of_spec=round(tf / spec, 3), clock_mhz=round(mhz))
    return out


def stored_traffic(case_name):
    """HBM bytes per stage-GEMM launch from the committed rocprofv3 counter
    summary, or None when the kernel source changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"traffic_gemm_dma_kernel_{case_name}.md")
    src = os.path.join(ROOT, "comm_overlapped_linear_amd", "csrc", "gemm.hip")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if line.startswith("- ") and ":" in line:
            k, v = line[2:].split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    if fields.get("gemm.hip sha256") != hashlib.sha256(open(src, "rb").read()).hexdigest():
        return None
    try:
        return float(fields["HBM bytes per launch"])
    except (KeyError, ValueError):
        return None


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max(i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas")
    except Exception:
        return os.cpu_count()


def profile_launches(fn, steps, peak):
    """Every launch of `steps` calls of fn(flags) with TPG_PROFILE (HIP events
    on each launch's own stream), grouped by kind: GEMM launches by flop
    count, against `peak` TFLOP/s; row kernels (negative work = HBM bytes)
    against the HBM peak. Kinds are listed largest first."""
    fn(tp.PROFILE)
    torch.cuda.synchronize()
    tp.profile_read()
    for _ in range(steps):
        fn(tp.PROFILE)
    torch.cuda.synchronize()
    recs = tp.profile_read()
    kinds = {}
    for ms_, work in recs:
        kinds.setdefault(work, []).append(ms_)
    out = []
    for work, v in sorted(kinds.items(), key=lambda kv: -abs(kv[0])):
        avg = float(np.mean(v))
        if work > 0:
            tf = work / (avg * 1e-3) / 1e12
            out.append(dict(kind="gemm", gflop=round(work / 1e9, 2), launches=len(v), avg_us=round(avg * 1e3, 2),
                            tflops=round(tf, 1), frac=round(tf / peak, 4)))
        else:
            gbs = -work / (avg * 1e-3) / 1e9
            out.append(dict(kind="hbm", mbytes=round(-work / 1e6, 1), launches=len(v), avg_us=round(avg * 1e3, 2),
                            gbs=round(gbs, 1), frac=round(gbs / HBM_PEAK_GBS, 4)))
    return out


def gemm_roofline(kinds, peak):
    """Sum of flops over sum of durations of the GEMM launches of one call."""
    g = [k for k in kinds if k["kind"] == "gemm"]
    fl = sum(k["gflop"] * k["launches"] for k in g)
    us = sum(k["avg_us"] * k["launches"] for k in g)
    tf = fl * 1e9 / (us * 1e-6) / 1e12 if us > 0 else 0.0
    return dict(bound="mfma", achieved=round(tf, 1), peak=peak, unit="TFLOP/s", frac=round(tf / peak, 4),
                by_launch=kinds)


# --------------------------------------------------------------------------- workloads
def setup_ag(case, extra_flags=0):
    inp = W.ag_inputs(case)
    slices = [dev(s) for s in inp["a_slices"]]
    b, c = dev(inp["b"]), dev(inp["c"]) if inp["c"] is not None else None
    nout = case.N // 2 if case.swiglu else case.N
    d = torch.empty((case.M, nout), dtype=torch.int16, device="cuda")
    kw = dict(M=case.M, N=case.N, K=case.K, rank=case.rank,
              dtype=tp.E4M3 if case.dtype == "e4m3" else tp.BF16,
              b_layout=tp.B_KN if case.b_layout == "kn" else tp.B_NK,
              epilogue=tp.EPI_SWIGLU if case.swiglu else tp.EPI_ALPHA_BETA,
              alpha=case.alpha, beta=case.beta)
    eb = 1 if case.dtype == "e4m3" else 2
    slice_bytes = case.m * case.K * eb
    # the unstaged call needs the most workspace (all P slices, then the K-split buffers)
    need = tp.stage_ag_workspace_size(tp.ag_args(slices, b, c, d, flags=tp.UNSTAGED, **kw))
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    # the same slices copied into one buffer: with TPG_NO_COPY the call then
    # makes the same launches as the staged call (one over all remote
    # stages), minus the deliveries
    whole = torch.cat(slices)
    views = [whole[i * case.m:(i + 1) * case.m] for i in range(case.P)]
    prepared_whole = tp.prepare_stage_ag(views, b, c, d, workspace=ws, flags=tp.NO_COPY, **kw)
    # --isolate-kernels (no deliveries, one stream) times those launches alone
    prepared = (prepared_whole if extra_flags & tp.NO_COPY
                else tp.prepare_stage_ag(slices, b, c, d, workspace=ws, flags=tp.UNSTAGED, **kw))

    def call(flags=0, groups=0):
        prepared._args.groups = groups
        prepared(flags=flags | extra_flags)

    def call_compute_only():
        prepared_whole(flags=tp.NO_COPY | extra_flags)

    def call_compute_only_ikg():
        prepared_whole(flags=tp.NO_COPY | tp.IN_KERNEL_GATES | extra_flags)

    side = torch.cuda.Stream()

    def deliveries(flags):
        """The P-1 deliveries alone, as the library issues them (tpg_deliver
        with the call's copy kind): ring order, back to back on one stream,
        recorded once into a graph so that replays time the copies rather
        than the host calls."""
        ring = [slices[(case.rank + t) % case.P] for t in range(1, case.P)]

        def issue():
            cur = torch.cuda.current_stream()
            side.wait_stream(cur)
            tp.deliver(ring, ws, nbytes=slice_bytes, flags=flags, stream=side)
            cur.wait_stream(side)
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            issue()
        return g.replay
    return inp, call, deliveries, dict(d=d, compute_only=call_compute_only, compute_only_ikg=call_compute_only_ikg)


CPU_SECONDS = 10.0      # bounded CPU sample: repeat the oracle call until this much time has passed
CPU_MAX_CALLS = 20


def cpu_baseline_ag_numpy(case, inp):
    """The numpy oracle, as it stands, on the same workload: whole calls
    repeated until about CPU_SECONDS of host time (at most CPU_MAX_CALLS),
    throughput from the total."""
    import oracle
    t0 = time.perf_counter()
    calls = 0
    while calls < CPU_MAX_CALLS and (calls == 0 or time.perf_counter() - t0 < CPU_SECONDS):
        oracle.gemm_ag(inp["a_slices"], inp["b"], inp["c"], case.alpha, case.beta, case.rank,
                       case.dtype, case.b_layout, swiglu=case.swiglu)
        calls += 1
    dt = time.perf_counter() - t0
    return dict(value=case.flop * calls / dt / 1e12, unit="TFLOP/s", cores=blas_threads(), kind="oracle",
                sample=f"the whole workload {calls} times ({case.flop / 1e9:.1f} GFLOP each, float64 numpy), "
                       f"{dt:.2f} s in total",
                cpu=cpu_model(), host_cpus=os.cpu_count())


CPP_SAMPLE_ROWS = 16     # rows per slice of the C++ oracle's bounded sample
CPP_MAX_CALLS = 200


def cpu_baseline_ag(case, inp):
    """The C++17 oracle (float64, OpenMP over output rows), as it stands, on a
    bounded sample of the workload: the first CPP_SAMPLE_ROWS rows of every
    slice against the whole B and K, repeated until about CPU_SECONDS of host
    time; throughput is the sample's flops over the time."""
    from oracle import cref
    cref.ensure_built()
    rows = min(CPP_SAMPLE_ROWS, case.m)
    slices = [np.ascontiguousarray(s[:rows]) for s in inp["a_slices"]]
    c = inp["c"]
    if c is not None:
        c = np.ascontiguousarray(np.concatenate([c[s * case.m:s * case.m + rows] for s in range(case.P)]))
    flop = 2.0 * case.P * rows * case.N * case.K
    t0 = time.perf_counter()
    calls = 0
    while calls < CPP_MAX_CALLS and (calls == 0 or time.perf_counter() - t0 < CPU_SECONDS):
        cref.gemm_ag(slices, inp["b"], c, case.alpha, case.beta, case.rank, case.dtype, case.b_layout,
                     swiglu=case.swiglu)
        calls += 1
    dt = time.perf_counter() - t0
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count()
    return dict(value=flop * calls / dt / 1e12, unit="TFLOP/s", cores=threads, kind="oracle",
                sample=f"C++17 oracle (float64, OpenMP): {rows} rows of each of the {case.P} slices "
                       f"({case.P * rows} of {case.M} rows, whole N and K; {flop / 1e9:.2f} GFLOP) "
                       f"{calls} times, {dt:.2f} s in total",
                cpu=cpu_model(), host_cpus=os.cpu_count())


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def bench_ag(case, args, detail):
    inp, call, deliveries, bufs = setup_ag(
        case, (tp.NO_COPY | tp.SERIAL_STAGES) if args.isolate_kernels else 0)
    dtype = "fp8_e4m3" if case.dtype == "e4m3" else "bf16"
    flop = case.flop

    ms = time_steps(lambda: call(0), args.steps, args.warmup)
    value = flop / (ms * 1e-3) / 1e12
    log(f"[{case.name}] staged (default issue): {ms * 1e3:.1f} us/step  {value:.1f} TFLOP/s")

    # dominant kernel: the stage GEMM, timed per launch with HIP events on its own stream
    call(tp.PROFILE)
    torch.cuda.synchronize()
    tp.profile_read()
    for _ in range(args.steps):
        call(tp.PROFILE)
    torch.cuda.synchronize()
    recs = tp.profile_read()
    kms = float(np.mean([r[0] for r in recs]))
    kflop = float(np.mean([r[1] for r in recs]))
    achieved = kflop / (kms * 1e-3) / 1e12            # = sum(flop) / sum(duration)
    peak = PEAK_TFLOPS[dtype]
    roofline = dict(bound="mfma", achieved=round(achieved, 2), peak=peak, unit="TFLOP/s",
                    frac=round(achieved / peak, 4), traffic=stored_traffic(case.name),
                    kernel="gemm_dma_kernel (stage runs of one call)", launches=len(recs),
                    launches_per_step=len(recs) // args.steps,
                    avg_launch_us=round(kms * 1e3, 2), flop_per_launch=kflop)
    # the same launches by kind (the local stage beside the deliveries, the
    # remote run over the delivered slices): flops, mean duration, rate
    kinds = {}
    for ms_, fl in recs:
        kinds.setdefault(fl, []).append(ms_)
    roofline["by_launch"] = [dict(gflop=round(fl / 1e9, 2), launches=len(v), avg_us=round(float(np.mean(v)) * 1e3, 2),
                                  tflops=round(fl / (float(np.mean(v)) * 1e-3) / 1e12, 1),
                                  frac=round(fl / (float(np.mean(v)) * 1e-3) / 1e12 / peak, 4))
                             for fl, v in sorted(kinds.items())]
    log(f"[{case.name}] stage GEMM launches: {kms * 1e3:.1f} us avg, {achieved:.1f} TFLOP/s "
        f"({len(recs)} launches, eager, HIP events on each launch's stream)")

    if not args.quick:
        t_compute = time_steps(bufs["compute_only"], args.steps, args.warmup)
        t_copy = time_steps(deliveries(0), args.steps, args.warmup)               # the AG default: copy kernel
        t_copy_sdma = time_steps(deliveries(tp.COPY_SDMA), args.steps, args.warmup)  # copy engines
        t_copy_shader = time_steps(deliveries(tp.COPY_SHADER), args.steps, args.warmup)  # runtime shader copy
        t_shader = time_steps(lambda: call(tp.COPY_SHADER), args.steps, args.warmup)
        t_unstaged = time_steps(lambda: call(tp.UNSTAGED), args.steps, args.warmup)
        t_per_stage = time_steps(lambda: call(0, case.P - 1), args.steps, args.warmup)
        t_sdma = time_steps(lambda: call(tp.COPY_SDMA), args.steps, args.warmup)
        t_graph = time_steps(lambda: call(tp.FORCE_GRAPH), args.steps, args.warmup)
        # the same stages one after another on one stream: deliveries, then each stage launch
        t_serial = time_steps(lambda: call(tp.SERIAL_STAGES), args.steps, args.warmup)
        # the staged call as one launch whose tiles wait in-kernel on chunk counters
        t_ikg = time_steps(lambda: call(tp.IN_KERNEL_GATES), args.steps, args.warmup)
        t_ikg_compute = time_steps(bufs["compute_only_ikg"], args.steps, args.warmup)
        hidden = 1.0 - (ms - t_compute) / t_copy if t_copy > 0 else None
        hidden_serial = (t_serial - ms) / t_copy if t_copy > 0 else None
        hidden_ikg = 1.0 - (t_ikg - t_ikg_compute) / t_copy if t_copy > 0 else None
        hidden_sdma = 1.0 - (t_sdma - t_compute) / t_copy_sdma if t_copy_sdma > 0 else None
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        flushed = time_flushed(lambda: call(0), max(args.steps, 100), 2, scratch)
        del scratch
        t_sus, n_sus = time_sustained(lambda: call(0))
        detail.update({
            "sustained_1s": dict(calls=n_sus, us=round(t_sus * 1e3, 2), tflops=round(flop / (t_sus * 1e-3) / 1e12, 1)),
            "us_staged": round(ms * 1e3, 2),
            "us_compute_only": round(t_compute * 1e3, 2),
            "us_deliveries_alone": round(t_copy * 1e3, 2),
            "hidden_fraction": None if hidden is None else round(hidden, 3),
            "us_serial_stages": round(t_serial * 1e3, 2),
            "hidden_fraction_serial": None if hidden_serial is None else round(hidden_serial, 3),
            "us_unstaged": round(t_unstaged * 1e3, 2),
            "us_one_gate_per_stage": round(t_per_stage * 1e3, 2),
            "us_staged_graph": round(t_graph * 1e3, 2),
            "us_in_kernel_gates": round(t_ikg * 1e3, 2),
            "us_in_kernel_gates_compute_only": round(t_ikg_compute * 1e3, 2),
            "hidden_fraction_in_kernel_gates": None if hidden_ikg is None else round(hidden_ikg, 3),
            "us_staged_copy_engines": round(t_sdma * 1e3, 2),
            "us_deliveries_alone_copy_engines": round(t_copy_sdma * 1e3, 2),
            "hidden_fraction_copy_engines": None if hidden_sdma is None else round(hidden_sdma, 3),
            "us_staged_runtime_shader_copy": round(t_shader * 1e3, 2),
            "us_deliveries_alone_runtime_shader_copy": round(t_copy_shader * 1e3, 2),
            "us_staged_l2_flushed": {k: round(v * 1e3, 2) for k, v in flushed.items()},
            "tflops_compute_only": round(flop / (t_compute * 1e-3) / 1e12, 1),
        })
        value_flushed = flop / (flushed["mean"] * 1e-3) / 1e12
        log(f"[{case.name}] detail: {json.dumps(detail)}")
    return dict(value=value, ms=ms, dtype=dtype, roofline=roofline, inp=inp,
                value_l2_flushed=None if args.quick else round(value_flushed, 2))


def bench_ffn(case, args):
    """The per-slot FFN layer forward (two slot streams), and its launches
    profiled on one stream (TPG_SERIAL_STAGES), so that each of the first
    GEMM (4096 x 15360 x 1280 per slot), the LayerNorm / SiLU pass (z read,
    h written: 6 H bytes per row) and the second GEMM (4096 x 1280 x 7680) is
    timed running alone."""
    inp = W.ffn_inputs(case)
    t = {k: dev(v) for k, v in inp.items()}
    y = torch.empty((case.PB, case.L, case.D), dtype=torch.int16, device="cuda")
    kw = dict(PB=case.PB, L=case.L, D=case.D, H=case.H, eps=case.eps)
    serial_ws = torch.empty(tp.ffn_slot_forward_workspace_size(tp.ffn_args(
        t["x"], t["w1"], t["b1"], t["wout"], t["bout"], t["gx"], t["bx"], t["gg"], t["bg"], y, flags=0, **kw)),
        dtype=torch.uint8, device="cuda")
    call = tp.prepare_ffn_slot_forward(t["x"], t["w1"], t["b1"], t["wout"], t["bout"], t["gx"], t["bx"],
                                       t["gg"], t["bg"], y, workspace=serial_ws, **kw)
    ms = time_steps(lambda: call(flags=0), max(3, args.steps // 2), 2)
    peak = PEAK_TFLOPS["bf16"]
    kinds = profile_launches(lambda f: call(flags=f | tp.SERIAL_STAGES), max(2, args.steps // 20), peak)
    call(flags=0)
    tf = case.flop / (ms * 1e-3) / 1e12
    return dict(us=round(ms * 1e3, 1), tflops=round(tf, 1), pct_bf16_peak=round(100 * tf / peak, 2),
                roofline_one_stream=gemm_roofline(kinds, peak))


def bench_ffn_backward(case, args):
    """Backward of the per-slot FFN layer at the workload size: every
    gradient (recomputes z and h, then dh, the LayerNorm / SiLU backward, the
    bias sums and the weight / input gradient GEMMs). Algorithmic flops: the
    recomputed first GEMM plus the four gradient GEMMs (2 x 2PB D 2H + 3 x 2PB D H
    per slot)."""
    inp = W.ffn_inputs(case)
    t = {k: dev(v) for k, v in inp.items()}
    dy = dev(W.ffn_upstream_grad(case))
    shapes = dict(dx=(case.PB, case.L, case.D), dw1=(case.L, case.D, 2 * case.H), db1=(case.L, 2 * case.H),
                  dwout=(case.L, case.H, case.D), dbout=(case.L, case.D), dgx=(case.H,), dbx=(case.H,),
                  dgg=(case.H,), dbg=(case.H,))
    grads = {k: torch.empty(s, dtype=torch.int16, device="cuda") for k, s in shapes.items()}
    call = tp.prepare_ffn_slot_backward(t["x"], t["w1"], t["b1"], t["wout"], t["gx"], t["bx"], t["gg"], t["bg"], dy,
                                        grads, PB=case.PB, L=case.L, D=case.D, H=case.H, eps=case.eps)
    ms = time_steps(call, max(3, args.steps // 5), 2)
    flop = case.L * (3 * 2.0 * case.PB * case.D * 2 * case.H + 2 * 2.0 * case.PB * case.D * case.H)
    return dict(us=round(ms * 1e3, 1), tflops=round(flop / (ms * 1e-3) / 1e12, 1), gflop=round(flop / 1e9, 1))


def bench_rs(case, args):
    inp = W.rs_inputs(case)
    a, b = dev(inp["a"]), dev(inp["b"])
    inc = [dev(x) if x is not None else None for x in inp["incoming"]]
    d = torch.empty((case.M, case.N), dtype=torch.int16, device="cuda")
    kw = dict(M=case.M, N=case.N, K=case.K, P=case.P, rank=case.rank,
              b_layout=tp.B_KN if case.b_layout == "kn" else tp.B_NK)
    need = tp.stage_rs_workspace_size(tp.rs_args(a, b, inc, d, flags=tp.UNSTAGED, **kw))
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    call = tp.prepare_stage_rs(a, b, inc, d, workspace=ws, **kw)
    steps = max(5, args.steps // 2)
    ms = time_steps(lambda: call(flags=0), steps, 3)
    mc = time_steps(lambda: call(flags=tp.NO_COPY), steps, 3)
    msh = time_steps(lambda: call(flags=tp.COPY_SHADER), steps, 3)
    msd = time_steps(lambda: call(flags=tp.COPY_SDMA), steps, 3)
    peak = PEAK_TFLOPS["bf16"]
    kinds = profile_launches(lambda f: call(flags=f), max(2, args.steps // 10), peak)
    call(flags=0)
    tf = case.flop / (ms * 1e-3) / 1e12
    return dict(us=round(ms * 1e3, 1), tflops=round(tf, 1), pct_bf16_peak=round(100 * tf / peak, 2),
                us_shader_copy=round(msh * 1e3, 1), us_copy_engines=round(msd * 1e3, 1),
                us_compute_only=round(mc * 1e3, 1),
                roofline=gemm_roofline(kinds, peak))


def bench_swiglu(case, args):
    inp = W.swiglu_inputs(case)
    xs = [dev(x) for x in inp["x_shards"]]
    w13, w2 = dev(inp["w13"]), dev(inp["w2"])
    h = torch.empty((case.M, case.F), dtype=torch.int16, device="cuda")
    out = torch.empty((case.M, case.D), dtype=torch.int16, device="cuda")
    ag = tp.prepare_stage_ag(xs, w13, None, h, M=case.M, N=2 * case.F, K=case.D,
                             rank=case.rank, b_layout=tp.B_KN, epilogue=tp.EPI_SWIGLU, alpha=1.0, beta=0.0)
    rs = tp.prepare_stage_rs(h, w2, None, out, M=case.M, N=case.D, K=case.F, P=case.P, rank=case.rank,
                             b_layout=tp.B_KN)

    def block(flags=0):
        ag(flags=flags)
        rs(flags=flags)
    ms = time_steps(block, max(5, args.steps // 2), 3)
    peak = PEAK_TFLOPS["bf16"]
    kinds = profile_launches(block, max(2, args.steps // 10), peak)
    block()
    tf = case.flop / (ms * 1e-3) / 1e12
    return dict(us=round(ms * 1e3, 1), tflops=round(tf, 1), pct_bf16_peak=round(100 * tf / peak, 2),
                roofline=gemm_roofline(kinds, peak))


def bench_column_duals(args):
    """The column-dual schedules at the e4m3 AG and bf16 RS workload shapes:
    rotating B (A local 8192 x 8192, B as 8 slices of 128 x 8192) and tiled B
    (8 column blocks of 1024 of the 8192 x 8192 x 3584 partial)."""
    out = {}
    c2 = W.AgCase("agb", M=8192, N=1024, K=8192, P=8, dtype="e4m3", dist="n05", beta=1.0)
    inp = W.ag_rotb_inputs(c2)
    a, bs, c = dev(inp["a"]), [dev(x) for x in inp["b_slices"]], dev(inp["c"])
    d = torch.empty((c2.M, c2.N), dtype=torch.int16, device="cuda")
    ag = tp.prepare_stage_ag(a, bs, c, d, M=c2.M, N=c2.N, K=c2.K, dtype=tp.E4M3, schedule=tp.ROTATE_B,
                             flags=tp.UNSTAGED)
    ms = time_steps(lambda: ag(flags=0), args.steps, args.warmup)
    mu = time_steps(lambda: ag(flags=tp.UNSTAGED), args.steps, args.warmup)
    out["ag_e4m3_rotb_p8_8192x1024x8192"] = dict(us=round(ms * 1e3, 1), tflops=round(c2.flop / (ms * 1e-3) / 1e12, 1),
                                                 us_unstaged=round(mu * 1e3, 1))
    c3 = W.RsCase("rsb", M=8192, N=8192, K=3584, P=8)
    inp = W.rs_tileb_inputs(c3)
    a, b = dev(inp["a"]), dev(inp["b"])
    inc = [dev(x) if x is not None else None for x in inp["incoming"]]
    d = torch.empty((c3.M, c3.N), dtype=torch.int16, device="cuda")
    rs = tp.prepare_stage_rs(a, b, inc, d, M=c3.M, N=c3.N, K=c3.K, P=c3.P, schedule=tp.TILE_B, flags=tp.UNSTAGED)
    steps = max(5, args.steps // 2)
    ms = time_steps(lambda: rs(flags=0), steps, 3)
    mu = time_steps(lambda: rs(flags=tp.UNSTAGED), steps, 3)
    out["rs_bf16_tileb_p8_8192x8192x3584"] = dict(us=round(ms * 1e3, 1), tflops=round(c3.flop / (ms * 1e-3) / 1e12, 1),
                                                  us_unstaged=round(mu * 1e3, 1))
    return out


WGRAD_BENCH = [W.WgCase("wgrad_bf16_p8_1024x8192_c8192", M=8192, N=1024, K=8192, P=8, gathered="x"),
               W.WgCase("wgrad_bf16_p8_w13_4096x3584_c8192", M=8192, N=4096, K=3584, P=8, gathered="g"),
               W.WgCase("wgrad_bf16_p8_w2_1792x4096_c8192", M=8192, N=1792, K=4096, P=8, gathered="x")]


def bench_wgrad(args):
    """Weight gradients of the backward pass: of the e4m3 all-gather shape
    (in bf16, X gathered) and of the SwiGLU block's w13 (G gathered) and w2
    (X gathered). Default call (one gathered launch), the staged chain
    (groups=1) and the GEMM alone over slices already in one buffer."""
    out = {}
    for case in WGRAD_BENCH:
        inp = W.wgrad_inputs(case)
        local, sl = dev(inp["local"]), [dev(x) for x in inp["slices"]]
        big = torch.cat(sl)
        whole = [big[i * case.m:(i + 1) * case.m] for i in range(case.P)]
        d = torch.empty((case.N, case.K), dtype=torch.int16, device="cuda")
        g = tp.GATHER_X if case.gathered == "x" else tp.GATHER_G
        kw = dict(M=case.M, N=case.N, K=case.K, gathered=g)
        need = max(tp.stage_wgrad_workspace_size(tp.wgrad_args(local, sl, d, groups=gr, **kw)) for gr in (0, 1))
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        call = tp.prepare_stage_wgrad(local, sl, d, workspace=ws, **kw)
        staged = tp.prepare_stage_wgrad(local, sl, d, workspace=ws, groups=1, **kw)
        gemm = tp.prepare_stage_wgrad(local, whole, d, flags=tp.UNSTAGED | tp.NO_COPY, **kw)
        steps = max(5, args.steps // 2)
        ms = time_steps(lambda: call(flags=0), steps, 3)
        ms_staged = time_steps(lambda: staged(flags=0), steps, 3)
        ms_gemm = time_steps(lambda: gemm(flags=tp.UNSTAGED | tp.NO_COPY), steps, 3)
        out[case.name] = dict(us=round(ms * 1e3, 1), tflops=round(case.flop / (ms * 1e-3) / 1e12, 1),
                              us_staged=round(ms_staged * 1e3, 1), us_gemm_only=round(ms_gemm * 1e3, 1),
                              tflops_gemm_only=round(case.flop / (ms_gemm * 1e-3) / 1e12, 1))
        del big, whole, local, sl, ws
    return out


def bench_qkv(args):
    """The fused QKV projection (several projections of one gathered input)
    of an 8B-class model at TP = 8: 8192 tokens, K = 4096, 512 + 128 + 128
    output columns per rank, bf16; weights apart (copied side by side each
    call) and back to back (read in place)."""
    case = W.QKV
    inp = W.ag_multi_inputs(case)
    slices = [dev(s) for s in inp["a_slices"]]
    apart = [dev(b) for b in inp["bs"]]
    whole = dev(np.concatenate(inp["bs"], axis=0))
    offs = np.cumsum([0] + list(case.ns))
    adjacent = [whole[offs[i]:offs[i + 1]] for i in range(len(case.ns))]
    ds = [torch.empty((case.M, n), dtype=torch.int16, device="cuda") for n in case.ns]
    kw = dict(M=case.M, K=case.K)

    def prepared(bs):
        need = max(tp.stage_ag_multi_workspace_size(tp.ag_multi_args(slices, bs, ds, flags=f, **kw))
                   for f in (0, tp.UNSTAGED))
        return tp.prepare_stage_ag_multi(slices, bs, ds, workspace=torch.empty(need, dtype=torch.uint8,
                                                                                device="cuda"), **kw)
    call, inplace = prepared(apart), prepared(adjacent)
    ms = time_steps(lambda: call(flags=0), args.steps, args.warmup)
    ms_in = time_steps(lambda: inplace(flags=0), args.steps, args.warmup)
    ms_un = time_steps(lambda: inplace(flags=tp.UNSTAGED), args.steps, args.warmup)
    return {case.name: dict(us=round(ms * 1e3, 1), tflops=round(case.flop / (ms * 1e-3) / 1e12, 1),
                            us_weights_adjacent=round(ms_in * 1e3, 1), us_unstaged=round(ms_un * 1e3, 1))}


def bench_small_ag(case, args):
    """A latency-bound staged call (0.07 GFLOP): microseconds are the figure
    of merit; the per-launch rates say how far its GEMMs are from peak."""
    inp, call, _, _ = setup_ag(case)
    ms = time_steps(lambda: call(0), args.steps, args.warmup)
    mu = time_steps(lambda: call(tp.UNSTAGED), args.steps, args.warmup)
    # the staged call as one launch carrying its deliveries, gated in-kernel
    mi = time_steps(lambda: call(tp.IN_KERNEL_GATES), args.steps, args.warmup)
    peak = PEAK_TFLOPS["bf16"]
    kinds = profile_launches(lambda f: call(f), max(5, args.steps // 5), peak)
    tf = case.flop / (ms * 1e-3) / 1e12
    return dict(us=round(ms * 1e3, 2), us_unstaged=round(mu * 1e3, 2), us_in_kernel_gates=round(mi * 1e3, 2),
                tflops=round(tf, 2), pct_bf16_peak=round(100 * tf / peak, 3), roofline=gemm_roofline(kinds, peak))


def bench_permutes(args):
    """dispatch_permute / combine_permute at the per-slot FFN's shapes: 8
    ranks' [512, 64, 1280] bf16 inputs into the dispatched [4096, 8, 1280],
    and back. Algorithmic bytes per call: every element read once and written
    once, 2 x 83.9 MB."""
    P, B, T, D = 8, 512, 64, 1280
    L = T // P
    srcs = [torch.randn((B, T, D), device="cuda").to(torch.bfloat16).view(torch.int16) for _ in range(P)]
    disp = [torch.empty((P * B, L, D), dtype=torch.int16, device="cuda") for _ in range(P)]
    back = torch.empty((B, T, D), dtype=torch.int16, device="cuda")
    nbytes = 2.0 * B * T * D * 2
    steps = max(10, args.steps)
    out = {}
    for name, fn in (("dispatch", lambda: tp.dispatch_permute(srcs, disp[0], rank=3, B=B, T=T, D=D, elem_bytes=2)),
                     ("combine", lambda: tp.combine_permute(disp, back, rank=3, B=B, T=T, D=D, elem_bytes=2))):
        ms = time_steps(fn, steps, 3)
        gbs = nbytes / (ms * 1e-3) / 1e9
        out[name] = dict(us=round(ms * 1e3, 2), gbs=round(gbs, 1), frac_hbm_peak=round(gbs / HBM_PEAK_GBS, 4),
                         mbytes=round(nbytes / 1e6, 1))
    return out


def overlap_point(staged, unstaged, serial, compute_only, deliveries, flop, steps, warmup):
    """Times of one sweep point (us) and the hidden fractions, negatives kept:
    (T_serial - T_staged) / T_deliveries with T_serial the same stages run one
    after another on one stream (the p04 statement's estimate), and
    1 - (T_staged - T_compute) / T_deliveries (T_serial taken as the sum of
    the isolated compute and deliveries)."""
    t = {k: time_steps(f, steps, warmup) for k, f in
         (("staged", staged), ("unstaged", unstaged), ("serial", serial), ("compute_only", compute_only),
          ("deliveries", deliveries))}
    hidden = 1.0 - (t["staged"] - t["compute_only"]) / t["deliveries"]
    hidden_serial = (t["serial"] - t["staged"]) / t["deliveries"]
    return dict(us_staged=round(t["staged"] * 1e3, 2), us_unstaged=round(t["unstaged"] * 1e3, 2),
                us_serial_stages=round(t["serial"] * 1e3, 2),
                us_compute_only=round(t["compute_only"] * 1e3, 2), us_deliveries_alone=round(t["deliveries"] * 1e3, 2),
                hidden_fraction_serial=round(hidden_serial, 3), hidden_fraction=round(hidden, 3),
                tflops_staged=round(flop / (t["staged"] * 1e-3) / 1e12, 1),
                staged_beats_unstaged=bool(t["staged"] < t["unstaged"]))


def bench_scale_sweep(args):
    """Where one-GPU staging hides its deliveries. The p04 statement's run
    flags scale the exchanged payload (comm scale) and the hidden width
    (compute scale). Read here for the all-gather forms: comm scale c
    multiplies the delivered bytes per flop by c at equal flops (c times the
    rows of each slice, 1/c of the output columns); compute scale k
    multiplies the output columns (flops) by k at equal delivered bytes.
    e4m3 all-gather: M = 8192 c, N = 1024 k / c, K = 8192. SwiGLU block:
    S = 1024 c tokens per shard, F = 1792 k / c, D = 4096 (its all-gather
    delivers the token shards; its reduce-scatter emits partials only)."""
    steps, warm = max(10, args.steps // 2), 3
    out = {}
    for c, k in ((1, 1), (2, 1), (1, 2), (2, 2)):
        case = W.AgCase(f"ag_e4m3_c{c}_k{k}", M=8192 * c, N=1024 * k // c, K=8192, P=8, dtype="e4m3",
                        dist="n05", c_dist="n01", beta=1.0)
        inp, call, deliveries, bufs = setup_ag(case)
        out[f"ag_e4m3_p8 comm x{c} compute x{k}"] = dict(
            M=case.M, N=case.N, K=case.K, delivered_mib=round(7 * case.m * case.K / 2 ** 20, 1),
            **overlap_point(lambda: call(0), lambda: call(tp.UNSTAGED), lambda: call(tp.SERIAL_STAGES),
                            bufs["compute_only"], deliveries(0), case.flop, steps, warm))
        log(f"[sweep] {case.name}: {out[f'ag_e4m3_p8 comm x{c} compute x{k}']}")
        del inp, call, deliveries, bufs
        torch.cuda.empty_cache()
    for c, k in ((1, 1), (2, 1), (1, 2), (2, 2)):
        case = W.SwigluCase(f"swiglu_c{c}_k{k}", S=1024 * c, D=4096, F=1792 * k // c, P=8)
        inp = W.swiglu_inputs(case)
        xs = [dev(x) for x in inp["x_shards"]]
        w13, w2 = dev(inp["w13"]), dev(inp["w2"])
        whole = torch.cat(xs)
        views = [whole[i * case.S:(i + 1) * case.S] for i in range(case.P)]
        h = torch.empty((case.M, case.F), dtype=torch.int16, device="cuda")
        o = torch.empty((case.M, case.D), dtype=torch.int16, device="cuda")
        akw = dict(M=case.M, N=2 * case.F, K=case.D, b_layout=tp.B_KN, epilogue=tp.EPI_SWIGLU, alpha=1.0, beta=0.0)
        need = tp.stage_ag_workspace_size(tp.ag_args(xs, w13, None, h, flags=tp.UNSTAGED, **akw))
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        ag = tp.prepare_stage_ag(xs, w13, None, h, workspace=ws, **akw)
        ag_in_place = tp.prepare_stage_ag(views, w13, None, h, flags=tp.NO_COPY, **akw)
        rs = tp.prepare_stage_rs(h, w2, None, o, M=case.M, N=case.D, K=case.F, P=case.P, b_layout=tp.B_KN)
        slice_bytes = case.S * case.D * 2
        side = torch.cuda.Stream()

        def deliveries():
            cur = torch.cuda.current_stream()
            side.wait_stream(cur)
            tp.deliver(xs[1:], ws, nbytes=slice_bytes, stream=side)
            cur.wait_stream(side)

        def block(flags):
            ag(flags=flags)
            rs(flags=flags & (tp.UNSTAGED | tp.SERIAL_STAGES))
        out[f"swiglu_p8 comm x{c} compute x{k}"] = dict(
            S=case.S, F=case.F, D=case.D, delivered_mib=round(7 * slice_bytes / 2 ** 20, 1),
            **overlap_point(lambda: block(0), lambda: block(tp.UNSTAGED), lambda: block(tp.SERIAL_STAGES),
                            lambda: (ag_in_place(flags=tp.NO_COPY), rs(flags=0)), deliveries, case.flop, steps, warm))
        log(f"[sweep] {case.name}: {out[f'swiglu_p8 comm x{c} compute x{k}']}")
        del xs, w13, w2, whole, views, h, o, ws, ag, ag_in_place, rs
        torch.cuda.empty_cache()
    return out


WORKLOADS = {"ag_e4m3_p8": W.C2, "ag_e4m3_p8_beta0": W.C2_BETA0, "ag_bf16_p2": W.C1}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="ag_e4m3_p8", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quick", action="store_true", help="headline and roofline only")
    ap.add_argument("--no-ffn", action="store_true", help="skip timing the per-slot FFN layer")
    ap.add_argument("--all", action="store_true",
                    help="also time the backward pass, the column-dual schedules and the fused QKV projection")
    ap.add_argument("--sweep", action="store_true",
                    help="delivered-bytes / compute scale sweep of the e4m3 all-gather and the SwiGLU block")
    ap.add_argument("--isolate-kernels", action="store_true",
                    help="run every call with no deliveries and one compute stream, so that each GEMM "
                         "dispatch runs alone (for per-dispatch hardware counters)")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="first run one plain 256 MiB copy (identity permute) whose HBM bytes are known, "
                         "to scale FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures the rank-local share on ONE GPU; peers are buffers in the same HBM. "
              "Runs on several GPUs are not supported: use --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    tp.lib()

    case = WORKLOADS[args.workload]
    detail = {}
    if args.calibration_copy:
        n = 256 << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty(n, dtype=torch.uint8, device="cuda")
        evict = torch.empty(4 * n, dtype=torch.uint8, device="cuda").fill_(2)   # push src out of L2 / MALL
        torch.cuda.synchronize()
        tp.dispatch_permute([src], dst, rank=0, B=1, T=1, D=n, elem_bytes=1)
        torch.cuda.synchronize()
        del src, dst, evict
    r = bench_ag(case, args, detail)
    probe = measure_mfma_peaks()
    detail["mfma_probe"] = probe
    log(f"[probe] {json.dumps(probe)}")
    measured = probe["e4m3" if r["dtype"] == "fp8_e4m3" else "bf16"]["tflops"]
    r["roofline"]["measured_peak"] = measured
    r["roofline"]["frac_of_measured_peak"] = round(r["roofline"]["achieved"] / measured, 4)
    if not args.quick:
        # the rest of the metric, every run: the other four workloads
        detail["ag_bf16_p2_256x256x512"] = bench_small_ag(W.C1, args)
        log(f"[c1] {json.dumps(detail['ag_bf16_p2_256x256x512'])}")
        detail["rs_bf16_p8_8192x8192x3584"] = bench_rs(W.C3, args)
        log(f"[c3] {json.dumps(detail['rs_bf16_p8_8192x8192x3584'])}")
        detail["swiglu_p8_s1024_d4096_f1792"] = bench_swiglu(W.C5, args)
        log(f"[c5] {json.dumps(detail['swiglu_p8_s1024_d4096_f1792'])}")
        if not args.no_ffn:
            detail["ffn_layer"] = bench_ffn(W.C4, args)
            log(f"[ffn] {json.dumps(detail['ffn_layer'])}")
        detail["permutes_ffn_shapes"] = bench_permutes(args)
        log(f"[permutes] {json.dumps(detail['permutes_ffn_shapes'])}")
    if args.all:
        if not args.no_ffn:
            detail["ffn_layer_backward"] = bench_ffn_backward(W.C4, args)
        detail.update(bench_column_duals(args))
        detail.update(bench_wgrad(args))
        detail.update(bench_qkv(args))
    if args.sweep:
        detail["scale_sweep"] = bench_scale_sweep(args)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_ag(case, r["inp"])
        log(f"[cpu] {cpu}")
        detail["cpu_baseline_numpy_oracle"] = cpu_baseline_ag_numpy(case, r["inp"])
        log(f"[cpu numpy] {detail['cpu_baseline_numpy_oracle']}")

    peak = PEAK_TFLOPS[r["dtype"]]
    out = {
        "metric": METRIC,
        "value": round(r["value"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": r["dtype"],
        "data": "synthetic",
        "config": {"workload": case.name, "M": case.M, "N": case.N, "K": case.K, "P": case.P,
                   "rank": case.rank, "alpha": case.alpha, "beta": case.beta, "b_layout": case.b_layout,
                   "pct_mfma_peak": round(100.0 * r["value"] / peak, 2),
                   "pct_measured_mfma_peak": round(100.0 * r["value"] / measured, 2),
                   "parallelism": "tp8 rank share"},
        "value_l2_flushed": r.get("value_l2_flushed"),
        "roofline": r["roofline"],
        "cpu_baseline": cpu,
        "detail": detail,
        "args": vars(args),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
