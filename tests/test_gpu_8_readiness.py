"""GPU tests of the readiness barrier, the gathered output and the run-time
corner cases of the schedules.

* Delay-injected == undelayed: every shard copy is held back (a bounded,
  host-set delay in the kernel that copies, or ahead of the copies on the
  side streams) after a run with other operands left their shards in the
  gathered image, so a consumer that did not wait for its strip would read
  the previous run's bytes.  Both executions, every schedule: the delayed
  run equals the undelayed one bit for bit, no wait runs out, and the step
  timeline shows the staged steps' GEMM work starting after the delay.
* The gathered output (dist_gemm_run_ag): equals the rotating operand bit
  for bit, and the products equal those of dist_gemm_run.
* A wait limit of zero: every wait runs out, the workgroup copies its strip
  itself, and the result is still exact.
* A reduce-scatter with beta = 0 and no C; alpha = 1/TP (the averaging
  reduce-scatter); options that rebuild the tables refused after a capture.
"""
import numpy as np
import pytest

import workloads
from gpu_helpers import check_full, empty_out, log, run_plan, to_gpu

pytestmark = pytest.mark.gpu

SCHEDS = ["AG_ROT_A", "AG_ROT_B", "RS_TILE_A_ROT_C", "RS_TILE_B_ROT_C"]


def _plan(w, x, options):
    import communication_tensor_gemm_amd as dg
    p = dg.Plan(w.M, w.N, w.K, w.L, w.TP, w.schedule, w.dtype)
    if w.in_dtype == "e4m3":
        p.set_scales(x.scale_a, x.scale_b)
    for k, v in options.items():
        p.set_option(k, v)
    return p


def _case(sched, dtype, M, N, K, L, TP, seed):
    beta = 1.0 if sched.startswith("RS") else 0.0
    return workloads.small_case(f"ready_{sched}_{dtype}_{M}x{N}x{K}_{seed}", sched, dtype, M, N, K, L,
                                TP, 1.0, beta, seed=seed)


def _args(w, dev):
    A, B, C = dev
    return A, B, (C if w.beta != 0.0 else None)


DELAY_US = 3000


@pytest.mark.parametrize("execution", [1, 0])
@pytest.mark.parametrize("sched,dtype,M,N,K,TP", [
    ("AG_ROT_A", "BF16_F32", 2048, 1536, 512, 8),
    ("AG_ROT_B", "E4M3_BF16", 1024, 3328, 512, 8),     # 416-column shards: strips straddle shards
    ("RS_TILE_A_ROT_C", "BF16_F32", 2048, 1024, 256, 8),
    ("RS_TILE_B_ROT_C", "F32", 512, 2048, 128, 4),
    ("AG_ROT_A", "BF16_BF16", 600, 520, 272, 4),       # no local strip: the first step claims its copy
])
def test_delay_injected_equals_undelayed(execution, sched, dtype, M, N, K, TP):
    import torch
    w = _case(sched, dtype, M, N, K, 1, TP, seed=71)
    x = workloads.generate(w)
    other = workloads.generate(_case(sched, dtype, M, N, K, 1, TP, seed=72))
    ref = run_plan(w, x, schedule="MONOLITHIC", TP=1)
    dev = (to_gpu(x.A), to_gpu(x.B), to_gpu(x.C))
    dev_o = (to_gpu(other.A), to_gpu(other.B), to_gpu(other.C))
    log("case", w.name, "execution", execution)
    with _plan(w, x, {"EXECUTION": execution, "STEP_TIMING": 2}) as p:
        # fill the gathered image with another run's shards
        D = empty_out(w)
        p.run(*_args(w, dev_o), D, w.alpha, w.beta)
        torch.cuda.synchronize()
        p.set_option("COPY_DELAY_US", DELAY_US)
        D = empty_out(w)
        p.run(*_args(w, dev), D, w.alpha, w.beta)
        torch.cuda.synchronize()
        assert torch.equal(D, ref), "delayed run != monolithic"
        assert p.device_errors() == 0
        tl = p.step_timeline()
        log("timeline", [tuple(round(v, 3) for v in t) for t in tl])
        delay_ms = DELAY_US / 1000.0
        steps = p.steps()
        for (copy_ms, begin_ms, end_ms), st in zip(tl, steps):
            if not st[2]:
                continue
            if execution == 0:
                assert copy_ms >= 0.9 * delay_ms, "a copy finished before the delay"
                assert begin_ms >= copy_ms - 0.05, "a step launch began before its copy"
            elif begin_ms >= 0:
                # a tile that reads a staged strip began only after the delayed copies
                assert begin_ms >= 0.9 * delay_ms, "a staged tile began before any copy"
                assert copy_ms >= 0.9 * delay_ms
        p.set_option("COPY_DELAY_US", 0)
        D2 = empty_out(w)
        p.run(*_args(w, dev), D2, w.alpha, w.beta)
        torch.cuda.synchronize()
        assert torch.equal(D2, ref)


@pytest.mark.parametrize("execution", [1, 0])
@pytest.mark.parametrize("sched,dtype,M,N,K,L,TP,shared", [
    ("AG_ROT_A", "BF16_F32", 1024, 768, 320, 1, 8, False),
    ("AG_ROT_A", "E4M3_BF16", 600, 520, 272, 2, 4, False),
    ("AG_ROT_A", "F32", 768, 512, 64, 3, 4, True),
    ("AG_ROT_B", "BF16_BF16", 512, 1664, 256, 1, 8, False),
    ("AG_ROT_B", "E4M3_F32", 384, 520, 128, 2, 4, False),
])
def test_gathered_output(execution, sched, dtype, M, N, K, L, TP, shared):
    import torch
    w = _case(sched, dtype, M, N, K, L, TP, seed=81)
    x = workloads.generate(w)
    if shared:
        x = workloads.Inputs(x.A[:1].copy(), x.B, x.C, x.scale_a, x.scale_b)
    A, B = to_gpu(x.A), to_gpu(x.B)
    opts = {"EXECUTION": execution, "SHARED_A": int(shared)}
    log("case", w.name, "execution", execution, "shared", shared)
    with _plan(w, x, opts) as p:
        D = empty_out(w)
        p.run(A, B, None, D, w.alpha, 0.0)
        src = A if sched == "AG_ROT_A" else B
        ag = torch.full_like(src, 0x55 if src.dtype != torch.float32 else float("nan"))
        Dg = empty_out(w)
        p.run_ag(A, B, None, Dg, ag, w.alpha, 0.0)
        torch.cuda.synchronize()
        assert torch.equal(ag.view(torch.uint8), src.view(torch.uint8)), "gathered operand differs"
        assert torch.equal(Dg, D), "products with a gathered output differ"
        assert p.device_errors() == 0
    if not shared:
        check_full(w, x, Dg)


def test_gathered_output_errors():
    import torch
    import communication_tensor_gemm_amd as dg
    A = torch.zeros(256 * 64, dtype=torch.int16, device="cuda")
    B = torch.zeros(256 * 64, dtype=torch.int16, device="cuda")
    D = torch.zeros(256 * 256, dtype=torch.float32, device="cuda")
    ag = torch.zeros_like(A)
    with dg.Plan(256, 256, 64, 1, 2, "RS_TILE_A_ROT_C", "BF16_F32") as p:
        with pytest.raises(dg.DistGemmError):
            p.run_ag(A, B, None, D, ag, 1.0, 0.0)
    with dg.Plan(256, 256, 64, 1, 2, "AG_ROT_A", "BF16_F32") as p:
        with pytest.raises(dg.DistGemmError):
            dg.dist_gemm_run_ag(p.handle, A, B, None, D, None, 1.0, 0.0)
        with pytest.raises(dg.DistGemmError):
            dg.dist_gemm_run_ag(p.handle, A, B, None, D, A, 1.0, 0.0)


@pytest.mark.parametrize("sched", SCHEDS)
def test_zero_wait_limit_copies_its_strip(sched):
    """Every wait runs out at once: the workgroup copies its strip into the
    gathered image itself; counted, and the result is exact."""
    import torch
    w = _case(sched, "BF16_F32", 1024, 1280, 256, 2, 4, seed=91)
    x = workloads.generate(w)
    ref = run_plan(w, x, schedule="MONOLITHIC", TP=1)
    dev = (to_gpu(x.A), to_gpu(x.B), to_gpu(x.C))
    log("case", w.name)
    with _plan(w, x, {"EXECUTION": 1, "WAIT_LIMIT_US": 0, "COPY_DELAY_US": 500}) as p:
        for i in range(2):
            D = empty_out(w)
            p.run(*_args(w, dev), D, w.alpha, w.beta)
            torch.cuda.synchronize()
            assert torch.equal(D, ref), f"run {i} with a zero wait limit"
        n0 = p.device_errors()
        log("timed-out waits:", n0)
        assert n0 > 0
        p.set_option("WAIT_LIMIT_US", 1000000)
        p.set_option("COPY_DELAY_US", 0)
        D = empty_out(w)
        p.run(*_args(w, dev), D, w.alpha, w.beta)
        torch.cuda.synchronize()
        assert p.device_errors() == n0
        assert torch.equal(D, ref)


@pytest.mark.parametrize("execution", [1, 0])
@pytest.mark.parametrize("sched", ["RS_TILE_A_ROT_C", "RS_TILE_B_ROT_C"])
def test_reduce_scatter_beta_zero_without_c(execution, sched):
    import torch
    w = workloads.small_case(f"rs_b0_{sched}", sched, "BF16_F32", 1024, 768, 192, 1, 4, 0.5, 0.0, seed=93)
    x = workloads.generate(w)
    A, B = to_gpu(x.A), to_gpu(x.B)
    log("case", w.name, "execution", execution)
    with _plan(w, x, {"EXECUTION": execution}) as p:
        D = empty_out(w)
        p.run(A, B, None, D, 0.5, 0.0)
        torch.cuda.synchronize()
        assert p.device_errors() == 0
    check_full(w, x, D)
    assert torch.equal(D, run_plan(w, x, schedule="MONOLITHIC", TP=1))


@pytest.mark.parametrize("execution", [1, 0])
@pytest.mark.parametrize("sched,TP", [("RS_TILE_A_ROT_C", 8), ("RS_TILE_B_ROT_C", 4)])
def test_reduce_scatter_average_alpha(execution, sched, TP):
    """The averaging reduce-scatter: alpha = 1/TP exactly, with beta = 1."""
    import torch
    w = workloads.small_case(f"rs_avg_{sched}", sched, "BF16_F32", 1024, 1024, 256, 1, TP, 1.0 / TP, 1.0,
                             seed=95)
    x = workloads.generate(w)
    log("case", w.name, "execution", execution)
    D = run_plan(w, x, options={"EXECUTION": execution})
    check_full(w, x, D)
    assert torch.equal(D, run_plan(w, x, schedule="MONOLITHIC", TP=1))


def test_table_options_refused_after_capture():
    """A captured run keeps its tables: options that rebuild them are refused
    afterwards and the graph keeps replaying correctly."""
    import torch
    import communication_tensor_gemm_amd as dg
    w = workloads.small_case("cap_lock", "AG_ROT_A", "BF16_F32", 1024, 512, 256, 1, 4, 1.0, 0.0, seed=97)
    x = workloads.generate(w)
    ref = run_plan(w, x, schedule="MONOLITHIC", TP=1)
    A, B = to_gpu(x.A), to_gpu(x.B)
    D = empty_out(w)
    s = torch.cuda.Stream()
    with _plan(w, x, {"EXECUTION": 1}) as p:
        p.set_option("QUEUES", 1)        # allowed before any capture
        p.set_option("QUEUES", 8)
        with torch.cuda.stream(s):
            p.run(A, B, None, D, 1.0, 0.0, stream=s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            p.run(A, B, None, D, 1.0, 0.0, stream=s)
        for opt, val in (("QUEUES", 1), ("COPY_CHUNK", 8192), ("COPY_AHEAD", 2), ("STEP_GROUP", 1),
                         ("SHARED_A", 1)):
            with pytest.raises(dg.DistGemmError) as ei:
                p.set_option(opt, val)
            assert ei.value.status == -3, opt
        p.set_option("WAIT_LIMIT_US", 500000)  # not a table option
        for i in range(2):
            D.fill_(0)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            _ = (A.float() * 2).sum().item()
            assert torch.equal(D, ref), f"replay {i}"


def _offset_like(t):
    """t's values in a fresh buffer that starts one element past an aligned
    address."""
    import torch
    flat = torch.empty(t.numel() + 8, dtype=t.dtype, device=t.device)
    v = flat[1:1 + t.numel()].view(t.shape)
    v.copy_(t)
    return v


@pytest.mark.parametrize("sched,dtype", [("AG_ROT_A", "BF16_F32"), ("AG_ROT_B", "BF16_BF16"),
                                         ("RS_TILE_A_ROT_C", "BF16_F32")])
def test_in_loop_copy_and_its_fallback(sched, dtype):
    """Shapes whose later steps are copied inside K loops (8192 x 4096 x 1024
    at TP=8: 16 slabs per tile, 512 tiles, so the first round of 256 reads
    steps 0-3 only).  With the rotating operand one element past an aligned
    address the in-loop copy is off and waiting and finished workgroups copy
    those steps; both runs, with and without a copy delay, equal the
    monolithic GEMM bit for bit, with no timed-out wait, and sampled outputs
    match the oracle."""
    import torch
    from gpu_helpers import check_sampled, sample_indices
    M, N = (8192, 4096) if sched != "AG_ROT_B" else (4096, 8192)
    w = _case(sched, dtype, M, N, 1024, 1, 8, seed=131)
    x = workloads.generate(w)
    A, B, C = to_gpu(x.A), to_gpu(x.B), to_gpu(x.C)
    ref = run_plan(w, x, schedule="MONOLITHIC", TP=1, dev=(A, B, C))
    rot = {"AG_ROT_A": 0, "AG_ROT_B": 1, "RS_TILE_A_ROT_C": 2}[sched]
    for off in (False, True):
        dev = [A, B, C]
        if off:
            dev[rot] = _offset_like(dev[rot])
        for delay in (0, 2000):
            log("case", w.name, "offset", off, "delay", delay)
            with _plan(w, x, {"EXECUTION": 1, "COPY_DELAY_US": delay}) as p:
                D = empty_out(w)
                p.run(*_args(w, tuple(dev)), D, w.alpha, w.beta)
                torch.cuda.synchronize()
                assert p.device_errors() == 0
            assert torch.equal(D, ref), (off, delay)
    rows = sample_indices(M, 8, 2, seed=3)
    cols = sample_indices(N, 8, 2, seed=4)
    check_sampled(w, x, ref, rows, cols)
