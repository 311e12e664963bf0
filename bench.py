#!/usr/bin/env python3
"""Benchmark of the TP-step GEMM on one MI355X.

One "step" of this benchmark is one dist_gemm_run: the whole TP-step schedule
(every shard copy and every step GEMM) over one set of resident synthetic
operands.  The default workload is the AllGather1D_TilingCD_RotatingA share
of one GPU at TP=8 of the <16384, 106496, 16384> GEMM that the Distributed
GEMM pull-request page times (bf16 in, fp32 accumulate and out; per step
2048 x 13312 x 16384).

Printed: one JSON line on stdout.  Progress goes to stderr.
  value        whole-run TFLOP/s = 2*M*N*K*L / (wall time per run)
  roofline     the step GEMM kernel: algorithmic flops of one launch over
               its mean duration, from HIP events recorded around every
               launch on the stream it runs on, over the timed region
  cpu_baseline the fp64 CPU oracle on a bounded sample of the same workload
  vendor_context  context only: torch's GEMM (hipBLASLt) on the monolithic
               shape on the same device
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "TFLOP/s + % MFMA peak of TP-step GEMM at TP=8 shard shapes, 1 MI355X"
# MI355X dense MFMA peaks (TFLOP/s) by input element type
PEAK = {"bf16": 2516.6, "f32": 157.3, "e4m3": 5033.2}
DEFAULT_CONFIG = "c3_ag_rot_a_bf16_tp8"
# the metric's other TP=8 shard shapes, timed in the same run as sub-records
SUB_CONFIGS = ["c4_rs_tile_a_rot_c_bf16_tp8", "c5_ag_rot_b_e4m3_tp8"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def pick_config(name):
    import workloads
    if name in workloads.CONFIGS:
        return workloads.CONFIGS[name]
    hits = [k for k in workloads.CONFIGS if k.startswith(name)]
    if len(hits) != 1:
        raise SystemExit(f"unknown or ambiguous config {name!r}; choose from {list(workloads.CONFIGS)}")
    return workloads.CONFIGS[hits[0]]


def to_gpu(arr):
    import numpy as np
    import torch
    if arr is None:
        return None
    if arr.dtype == np.uint16:
        arr = arr.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


class SclkSampler:
    """Shader clock read from the amdgpu sysfs level table (pp_dpm_sclk: the
    current level is marked '*') every few milliseconds on a background
    thread.  The reported level lags the load by a fraction of a second, so it
    is sampled over a sustained phase of the same runs (see sustained_sclk),
    not over the short timed region.  Unavailable (no readable table, or
    several GPUs without a match for device 0) -> no samples."""

    def __init__(self):
        import glob
        self.path = None
        self.samples = []
        paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        if len(paths) > 1:
            try:
                import torch
                bus = str(getattr(torch.cuda.get_device_properties(0), "pci_bus_id", "")).lower()
                paths = [q for q in paths if bus and bus in os.path.realpath(os.path.dirname(q)).lower()]
            except Exception:
                paths = []
        if len(paths) == 1 and self._read(paths[0]) is not None:
            self.path = paths[0]

    @staticmethod
    def _read(path):
        try:
            with open(path) as f:
                for line in f:
                    if line.rstrip().endswith("*"):
                        return float(line.split(":")[1].strip().rstrip("*").strip().lower().rstrip("mhz"))
        except Exception:
            return None
        return None

    def __enter__(self):
        import threading
        self._stop = threading.Event()
        self._t = None
        if self.path:
            def loop():
                while not self._stop.is_set():
                    v = self._read(self.path)
                    if v is not None:
                        self.samples.append(v)
                    self._stop.wait(0.005)
            self._t = threading.Thread(target=loop, daemon=True)
            self._t.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._t:
            self._t.join()
        return False

    def summary(self, skip_fraction=0.0):
        v = self.samples[int(len(self.samples) * skip_fraction):]
        if not v:
            return None
        v = sorted(v)
        return {"median": v[len(v) // 2], "min": v[0], "max": v[-1], "samples": len(v),
                "source": "pp_dpm_sclk"}


def sustained_sclk(plan, args_run, seconds=1.5):
    """Run the plan back to back for about `seconds` and sample the shader
    clock; the second half of the samples (after the reported level has
    settled) is summarised.  None where the clock cannot be read."""
    import torch
    sampler = SclkSampler()
    if not sampler.path:
        return None
    with sampler:
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            for _ in range(10):
                plan.run(*args_run)
            torch.cuda.synchronize()
    out = sampler.summary(skip_fraction=0.5)
    if out:
        out["phase_s"] = seconds
    return out


def timed_runs(plan, args_run, steps, warmup, timing_runs, sampler=None, name="run"):
    import torch
    for _ in range(warmup):
        plan.run(*args_run)
    torch.cuda.synchronize()
    if timing_runs:
        plan.set_option("STEP_TIMING", steps)
    # per-run events on the stream the runs are enqueued on (the null stream)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    torch.cuda.synchronize()
    import contextlib
    with (sampler if sampler is not None else contextlib.nullcontext()):
        t0 = time.perf_counter()
        for b, e in evs:
            ROCTX.push(name)
            b.record()
            plan.run(*args_run)
            e.record()
            ROCTX.pop()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    step_ms = plan.step_times() if timing_runs else []
    run_ms = sorted(b.elapsed_time(e) for b, e in evs)
    stats = {"mean": sum(run_ms) / len(run_ms), "median": run_ms[len(run_ms) // 2], "min": run_ms[0]}
    return (t1 - t0) / steps * 1e3, step_ms, stats


def flushed_runs(plan, args_run, steps, nbytes=1 << 30):
    """Cold-cache timing: before each run a 1 GiB scratch buffer is written (the
    last-level cache is 256 MB), and HIP events bracket the run alone."""
    import torch
    scratch = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i, (b, e) in enumerate(evs):
        scratch.fill_(float(i))
        b.record()
        plan.run(*args_run)
        e.record()
    torch.cuda.synchronize()
    ms = sorted(b.elapsed_time(e) for b, e in evs)
    del scratch
    return {"mean": sum(ms) / len(ms), "median": ms[len(ms) // 2], "min": ms[0]}


def cpu_baseline(w, x, rows_per_block):
    """The oracle (as it stands) on a sample: rows_per_block rows from each of
    the S row blocks (or S x rows_per_block rows for column schedules), all N
    columns, every step visited."""
    import numpy as np
    from oracle import gemm
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = None
    S = w.TP if w.schedule != "MONOLITHIC" else 1
    if w.schedule in ("AG_ROT_A", "RS_TILE_A_ROT_C"):
        blk = w.M // S
        rows = np.concatenate([np.arange(s * blk, s * blk + min(rows_per_block, blk))
                               for s in range(S)])
    else:
        rows = np.arange(min(w.M, rows_per_block * S))
    cols = np.arange(w.N)
    t0 = time.perf_counter()
    gemm.dist_gemm_sampled(x.A, x.B, x.C, w.alpha, w.beta, w.schedule, S, w.in_dtype,
                           w.out_dtype, rows, cols, x.scale_a, x.scale_b)
    dt = time.perf_counter() - t0
    flops = 2.0 * len(rows) * len(cols) * w.K
    cores = len(os.sched_getaffinity(0))
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads or cores,
            "host_cores": cores, "kind": "oracle", "seconds": dt,
            "sample": f"{len(rows)} of {w.M} rows x all {w.N} columns x K={w.K} "
                      f"({flops / 1e12:.3f} TFLOP), fp64 numpy matmul per step"}


def parity_spot_check(w, x, D):
    import numpy as np
    import torch
    from oracle import codecs, gemm, parity
    g = np.random.default_rng(0)
    rows = np.unique(np.concatenate([g.integers(0, w.M, 48), [0, w.M - 1]]))
    cols = np.unique(np.concatenate([g.integers(0, w.N, 48), [0, w.N - 1]]))
    S = w.TP if w.schedule != "MONOLITHIC" else 1
    Ds, rn, cn = gemm.dist_gemm_sampled(x.A, x.B, x.C, w.alpha, w.beta, w.schedule, S,
                                        w.in_dtype, w.out_dtype, rows, cols, x.scale_a,
                                        x.scale_b)
    sub = D[0].index_select(0, torch.from_numpy(rows).cuda()).index_select(
        1, torch.from_numpy(cols).cuda()).cpu().numpy()
    got = sub.astype(np.float64) if w.out_dtype == "f32" else codecs.bf16_to_f64(sub.view(np.uint16))
    c = None if w.beta == 0 else codecs.decode(x.C[0][np.ix_(rows, cols)], w.out_dtype)
    ok, mx, tight, _ = parity.check(got, Ds, rn, cn, w.alpha, w.beta, c, w.in_dtype, w.out_dtype)
    return {"ok": bool(ok and tight), "max_normalised_err": mx, "n": int(got.size)}


KERNEL_SOURCES = ["communication_tensor_gemm_amd/csrc/distgemm.hip",
                  "communication_tensor_gemm_amd/csrc/gemm_tile.h",
                  "communication_tensor_gemm_amd/csrc/gemm_launch.h",
                  "communication_tensor_gemm_amd/csrc/fused_run.h",
                  "communication_tensor_gemm_amd/csrc/gemm_mfma16.hip",
                  "communication_tensor_gemm_amd/csrc/gemm_mfma_f8.hip",
                  "communication_tensor_gemm_amd/build.py"]
TRAFFIC_FILE = "profiles/fused_run_kernel_hbm_traffic.txt"


def kernel_source_hash():
    """Hash of the kernel sources' code: comments, blank lines and trailing
    blanks removed, so that a comment edit leaves a recorded measurement
    valid and any code change invalidates it."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        text = open(os.path.join(ROOT, f), encoding="utf-8").read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        # // comments (a "//" inside a string literal is not one: the sources have none)
        text = re.sub(r"//[^\n]*", "", text)
        lines = [l.rstrip() for l in text.splitlines()]
        h.update("\n".join(l for l in lines if l).encode())
    return h.hexdigest()[:16]


def recorded_traffic(workload):
    """HBM bytes per step-kernel launch from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE record, if it was taken on the current kernel sources."""
    path = os.path.join(ROOT, TRAFFIC_FILE)
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = line.split("=", 1)
            rec[k.strip()] = v.strip()
    if rec.get("kernel_sources_sha256_16") != kernel_source_hash():
        return None
    v = rec.get(f"{workload}.bytes_per_launch")
    return float(v) if v else None


def calibrate_copy(nbytes, reps):
    """A plain device-to-device copy of known size (the scale reference for
    the HBM byte counters): reps copies of nbytes each."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": nbytes, "reps": reps}), flush=True)


class Roctx:
    """roctx ranges around every timed run (rocprofv3 --marker-trace shows
    them), through the ROCm tracer library if it loads; otherwise a no-op."""

    def __init__(self):
        import ctypes
        self.lib = None
        for name in ("libroctx64.so", "/opt/rocm/lib/libroctx64.so"):
            try:
                self.lib = ctypes.CDLL(name)
                self.lib.roctxRangePushA.argtypes = [ctypes.c_char_p]
                break
            except OSError:
                continue

    def push(self, name: str):
        if self.lib:
            self.lib.roctxRangePushA(name.encode())

    def pop(self):
        if self.lib:
            self.lib.roctxRangePop()


ROCTX = Roctx()


def make_plan(w, x, args, options=None):
    import communication_tensor_gemm_amd as dg
    plan = dg.Plan(w.M, w.N, w.K, w.L, w.TP, w.schedule, w.dtype)
    if w.in_dtype == "e4m3":
        plan.set_scales(x.scale_a, x.scale_b)
    opts = {"COMPUTE_STREAMS": args.compute_streams, "COPY_ENGINE": args.copy_engine,
            "COPY_STREAMS": args.copy_streams, "STEP_GROUP": args.step_group,
            "EXECUTION": args.execution, "QUEUES": args.queues, "COPY_CHUNK": args.copy_chunk,
            "COPY_AHEAD": args.copy_ahead, "HALF_TILES": args.half_tiles}
    opts.update(options or {})
    for k, v in opts.items():
        plan.set_option(k, v)
    return plan


def copy_alone_ms(w, A, B, C, reps=5):
    """The rotation's bytes (the S-1 staged shards) moved by a plain device
    copy on an otherwise idle GPU: what the copies cost when nothing runs
    beside them."""
    import torch
    S = w.TP
    if w.schedule == "AG_ROT_A":
        src = A.view(w.L, S, -1)
    elif w.schedule == "AG_ROT_B":
        src = B.view(w.L, S, -1)
    elif w.schedule == "RS_TILE_A_ROT_C":
        src = C.view(w.L, S, -1)
    else:
        src = C.view(w.L * w.M, S, -1)
    src = src[:, 1:]
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    b, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    b.record()
    for _ in range(reps):
        dst.copy_(src)
    e.record()
    torch.cuda.synchronize()
    ms = b.elapsed_time(e) / reps
    nbytes = src.numel() * src.element_size()
    del dst
    return {"ms": round(ms, 4), "bytes": nbytes, "GB_per_s": round(2 * nbytes / (ms * 1e-3) / 1e9, 1),
            "what": "the S-1 staged shards copied by a plain device copy (torch copy_), GPU otherwise idle"}


def vendor_context(w, mono_ms, reps=20):
    """Context only, outside the product: the vendor library (hipBLASLt
    through torch) on the monolithic shape, same device, random operands of
    the input type.  bf16 and fp32: torch.matmul(A, B^T) (bf16 output for
    bf16 inputs, no C); e4m3: torch._scaled_mm with unit scales, bf16 output.
    Not a like-for-like comparison where the output type or the C read
    differ; reported so that the GEMM kernel can be read against the
    device's own library."""
    import torch
    out = {}
    try:
        M, N, K = w.M, w.N, w.K
        g = torch.Generator(device="cuda")
        g.manual_seed(0)
        if w.in_dtype == "e4m3":
            A = (torch.randn(M, K, device="cuda", generator=g) * 64).to(torch.float8_e4m3fn)
            B = (torch.randn(N, K, device="cuda", generator=g) * 64).to(torch.float8_e4m3fn)
            one = torch.ones((), device="cuda")
            fn = lambda: torch._scaled_mm(A, B.t(), scale_a=one, scale_b=one, out_dtype=torch.bfloat16)  # noqa: E731
            what = "torch._scaled_mm, e4m3 in, bf16 out"
        else:
            dt = torch.bfloat16 if w.in_dtype == "bf16" else torch.float32
            A = torch.randn(M, K, device="cuda", generator=g).to(dt)
            B = torch.randn(N, K, device="cuda", generator=g).to(dt)
            fn = lambda: torch.matmul(A, B.t())  # noqa: E731
            what = f"torch.matmul, {w.in_dtype} in and out, no C"
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out = {"what": what, "ms": round(ms, 4), "tflops": round(w.flops / (ms * 1e-3) / 1e12, 2)}
        if mono_ms:
            out["our_monolithic_over_it"] = round(ms / mono_ms, 4)
    except Exception as e:  # context only: never fails the bench
        out = {"error": f"{type(e).__name__}: {str(e)[:200]}"}
    finally:
        A = B = None
        torch.cuda.empty_cache()
    return out


def measure(w, args, headline):
    """Time one workload: the schedule, its monolithic GEMM, parity, the
    rotation's copy alone; the sustained clock for the headline only."""
    import numpy as np
    import torch

    import workloads
    S = w.TP if w.schedule != "MONOLITHIC" else 1
    log(f"[bench] workload {w.name}: {w.schedule} {w.dtype} M={w.M} N={w.N} K={w.K} TP={w.TP}")
    t = time.perf_counter()
    x = workloads.generate(w)
    log(f"[bench] inputs generated in {time.perf_counter() - t:.1f}s")
    A, B, C = to_gpu(x.A), to_gpu(x.B), to_gpu(x.C)
    out_dt = torch.float32 if w.out_dtype == "f32" else torch.int16
    D = torch.empty((w.L, w.M, w.N), dtype=out_dt, device="cuda")
    plan = make_plan(w, x, args)
    run_args = (A, B, C if w.beta != 0 else None, D, w.alpha, w.beta)
    log(f"[bench] timing {args.steps} runs after {args.warmup} warmup runs")
    fused = args.execution == 1 and S > 1
    # One launch per run: the per-run events on the launch's stream time the
    # launch itself, so the timed runs carry no per-step instrumentation;
    # the step timeline comes from two more runs afterwards.
    ms, step_ms, run_stats = timed_runs(plan, run_args, args.steps, args.warmup, not fused, name=w.name)
    value = w.flops / (ms * 1e-3) / 1e12
    peak = PEAK[w.in_dtype]
    if fused:
        _, _, _ = timed_runs(plan, run_args, 2, 0, True, name=w.name + ".timeline")
    timeline = plan.step_timeline()
    if fused:
        n_launch = 1
        avg_launch_ms = run_stats["mean"]
        busy = avg_launch_ms
    else:
        # Steps merged into one launch share its duration equally; the time at
        # least one step GEMM ran (overlapping launches on two compute streams
        # stretch each one's span) comes from the last run's timeline.
        spans = sorted({(b, e) for _, b, e in timeline})
        busy, cur = 0.0, None
        for b, e in spans:
            if cur is None or b > cur[1]:
                if cur is not None:
                    busy += cur[1] - cur[0]
                cur = [b, e]
            else:
                cur[1] = max(cur[1], e)
        busy += cur[1] - cur[0]
        n_launch = len(spans)
        avg_launch_ms = float(np.mean(step_ms)) * S / n_launch
    flops_per_launch = w.flops / n_launch
    achieved = flops_per_launch / (avg_launch_ms * 1e-3) / 1e12
    achieved_busy = w.flops / (busy * 1e-3) / 1e12
    log(f"[bench] {ms:.3f} ms/run, {value:.1f} TFLOP/s ({100 * value / peak:.1f}% of peak); "
        f"{n_launch} launches/run, per-launch {achieved:.1f} TFLOP/s")
    flushed = None
    if args.flush:
        plan.set_option("STEP_TIMING", 0)
        fl = flushed_runs(plan, run_args, args.steps)
        flushed = {"run_ms": {k: round(v, 4) for k, v in fl.items()},
                   "tflops_mean": round(w.flops / (fl["mean"] * 1e-3) / 1e12, 2),
                   "what": "1 GiB scratch written before each run (cold last-level cache); events around the run"}
        log(f"[bench] flushed-cache runs: {flushed}")
    parity = parity_spot_check(w, x, D)
    log(f"[bench] parity spot check: {parity}")
    mono = None
    if not args.no_mono:
        import communication_tensor_gemm_amd as dg
        with dg.Plan(w.M, w.N, w.K, w.L, 1, "MONOLITHIC", w.dtype) as mp:
            if w.in_dtype == "e4m3":
                mp.set_scales(x.scale_a, x.scale_b)
            mp.set_option("HALF_TILES", args.half_tiles)
            mono_ms, mono_steps, mono_stats = timed_runs(mp, run_args, args.steps, args.warmup, True,
                                                         name=w.name + ".monolithic")
        mono = {"ms": round(mono_ms, 4), "tflops": round(w.flops / (mono_ms * 1e-3) / 1e12, 2),
                "kernel_ms": round(float(np.mean(mono_steps)), 4),
                "run_ms": {k: round(v, 4) for k, v in mono_stats.items()},
                "exposed_overhead": round(ms / mono_ms - 1.0, 4)}
        log(f"[bench] monolithic {mono_ms:.3f} ms ({mono['tflops']:.1f} TFLOP/s); "
            f"schedule overhead {100 * mono['exposed_overhead']:.1f}%")
    copy_alone = copy_alone_ms(w, A, B, C) if S > 1 else None
    log(f"[bench] rotation copy alone: {copy_alone}")
    vendor = None
    if not args.no_vendor and w.L == 1:
        vendor = vendor_context(w, mono["ms"] if mono else None)
        log(f"[bench] vendor library on the monolithic shape (context): {vendor}")
    wait_timeouts = plan.device_errors()
    sclk_stats = None
    if headline:
        # after both timed comparisons, so that neither starts from a GPU
        # this phase has warmed
        plan.set_option("STEP_TIMING", 0)
        sclk_stats = sustained_sclk(plan, run_args)
        log(f"[bench] shader clock while the runs repeat: {sclk_stats}")
    plan.close()
    del A, B, C, D
    torch.cuda.empty_cache()
    rec = {
        "value": round(value, 2), "unit": "TFLOP/s", "ms_per_step": round(ms, 4),
        "pct_mfma_peak": round(100 * value / peak, 2),
        "config": {"workload": w.name, "schedule": w.schedule, "M": w.M, "N": w.N, "K": w.K,
                   "L": w.L, "TP": w.TP, "in": w.in_dtype, "out": w.out_dtype,
                   "alpha": w.alpha, "beta": w.beta},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": recorded_traffic(w.name),
                     "kernel": ("gemm_tn_kernel (step GEMM launches)" if args.execution == 0 else
                                "fused_run_kernel (one launch: shard copies and all tiles)"),
                     "avg_launch_ms": round(avg_launch_ms, 4),
                     "flops_per_launch": flops_per_launch, "launches_per_run": n_launch,
                     "gemm_busy_ms": round(busy, 4),
                     "achieved_while_busy": round(achieved_busy, 2)},
        "timeline_last_run": {"copy_done_ms": [round(t[0], 4) for t in timeline],
                              "gemm_begin_ms": [round(t[1], 4) for t in timeline],
                              "gemm_end_ms": [round(t[2], 4) for t in timeline]},
        "run_ms": {k: round(v, 4) for k, v in run_stats.items()},
        "monolithic": mono,
        # the single launch computes the monolithic tile grid, so without its
        # copies it is the monolithic kernel: t_nocopy is its time
        "t_nocopy_ms": mono["ms"] if (mono and args.execution == 1) else None,
        "t_copy_only": copy_alone,
        "flushed": flushed,
        "parity": parity,
        "device_wait_timeouts": wait_timeouts,
        "vendor_context": vendor,
    }
    return rec, x, sclk_stats


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    # 100 timed runs per workload, the CUTLASS example page's default iteration count
    ap.add_argument("--steps", type=int, default=100)
    # untimed runs before each timed set: the clock dips for the first tens of
    # runs of a sudden sustained load and recovers after about a hundred
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--config", default=DEFAULT_CONFIG)
    ap.add_argument("--compute-streams", type=int, default=2)
    ap.add_argument("--copy-engine", type=int, default=2,
                    help="0 SDMA, 1 runtime device copy, 2 library copy kernel (default)")
    ap.add_argument("--copy-streams", type=int, default=2, help="side streams for the shard copies (1..8)")
    ap.add_argument("--step-group", type=int, default=2, help="consecutive staged steps per GEMM launch")
    ap.add_argument("--execution", type=int, default=1,
                    help="0 = step launches + side-stream copies, 1 = one persistent launch per run")
    ap.add_argument("--queues", type=int, default=8, help="work queues of the single launch (1 or 8)")
    ap.add_argument("--copy-chunk", type=int, default=2 << 20, help="bytes per copy item of the single launch")
    ap.add_argument("--copy-ahead", type=int, default=0,
                    help="segments of the single launch whose tiles claim a copy quota before their GEMM")
    ap.add_argument("--half-tiles", type=int, default=1,
                    help="1: a last round of tiles that fills at most half the CUs runs as half-height tiles")
    ap.add_argument("--cpu-rows", type=int, default=2048,
                    help="oracle sample: rows per step block for the CPU baseline")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU baseline")
    ap.add_argument("--no-mono", action="store_true", help="skip the monolithic comparison")
    ap.add_argument("--no-vendor", action="store_true",
                    help="skip the vendor-library context timing of the monolithic shape")
    ap.add_argument("--flush", action="store_true",
                    help="also time runs with a 1 GiB scratch write before each (cold caches), reported separately")
    ap.add_argument("--no-sub", action="store_true",
                    help="time only --config, not the other TP=8 workloads")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run plain copies of BYTES (HBM counter calibration) and exit")
    args = ap.parse_args()

    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy, 3)
        return

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): this build "
              "times one GPU's share of the TP schedule; multi-GPU runs are not part of it.",
              file=sys.stderr, flush=True)
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    w = pick_config(args.config)
    rec, x, sclk_stats = measure(w, args, headline=True)
    subs = {}
    if not args.no_sub:
        for name in [n for n in SUB_CONFIGS if pick_config(n).name != w.name]:
            sub, _, _ = measure(pick_config(name), args, headline=False)
            subs[sub["config"]["workload"]] = sub

    cpu = None
    if not args.no_cpu:
        log(f"[bench] CPU oracle baseline on a sample ({args.cpu_rows} rows per step block)")
        cpu = cpu_baseline(w, x, args.cpu_rows)
        log(f"[bench] CPU oracle {cpu['value'] * 1e3:.1f} GFLOP/s in {cpu['seconds']:.1f}s")

    dtype_name = {"bf16": "bf16", "f32": "f32", "e4m3": "e4m3"}[w.in_dtype]
    peak = PEAK[w.in_dtype]
    config = dict(rec["config"])
    config.update({"compute_streams": args.compute_streams,
                   "copy_engine": ["sdma", "runtime_device_copy", "copy_kernel"][args.copy_engine],
                   "copy_streams": args.copy_streams, "step_group": args.step_group,
                   "execution": ["step_launches", "single_launch"][args.execution],
                   "queues": args.queues, "copy_chunk": args.copy_chunk,
                   "copy_ahead": args.copy_ahead, "half_tiles": args.half_tiles})
    out = {
        "metric": METRIC,
        "value": rec["value"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": rec["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype_name,
        "data": "synthetic",
        "config": config,
        "pct_mfma_peak": rec["pct_mfma_peak"],
        # the same rate against the peak at the shader clock measured while
        # the same runs execute back to back (the published peak assumes 2400 MHz)
        "sclk_mhz": sclk_stats,
        "pct_mfma_peak_at_sclk": (round(100 * rec["value"] / (peak * sclk_stats["median"] / 2400.0), 2)
                                  if sclk_stats else None),
        "roofline": rec["roofline"],
        "timeline_last_run": rec["timeline_last_run"],
        "run_ms": rec["run_ms"],
        "monolithic": rec["monolithic"],
        "t_nocopy_ms": rec["t_nocopy_ms"],
        "t_copy_only": rec["t_copy_only"],
        "flushed": rec["flushed"],
        "parity": rec["parity"],
        "device_wait_timeouts": rec["device_wait_timeouts"],
        "vendor_context": rec["vendor_context"],
        "cpu_baseline": cpu,
        # the other TP=8 shard shapes of the metric, measured the same way in
        # the same process (not part of value)
        "other_workloads": subs,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
