"""GPU tests of the single-launch execution (DIST_GEMM_OPT_EXECUTION = 1): one
persistent launch copies the staged shards in pieces and computes the tiles
of the monolithic tile grid, each tile of a staged strip waiting on that
strip's device-side counter.

Every case is checked against the fp64 oracle and, bitwise, against the
step-launch execution of the same plan (same kernel tile, same K order), and
no device-side wait may run out.  Runs repeat on one plan with new operands,
interleave plans, overlap plans on two streams, and replay from a HIP graph,
so that the counters are shown to start from zero every time.
"""
import numpy as np
import pytest

import workloads
from gpu_helpers import check_full, check_sampled, empty_out, log, run_plan, sample_indices, to_gpu

pytestmark = pytest.mark.gpu

SCHEDS = ["AG_ROT_A", "AG_ROT_B", "RS_TILE_A_ROT_C", "RS_TILE_B_ROT_C"]
DTYPES = ["F32", "BF16_F32", "BF16_BF16", "E4M3_BF16", "E4M3_F32"]
FUSED = {"EXECUTION": 1}


def _plan(w, x, options):
    import communication_tensor_gemm_amd as dg
    p = dg.Plan(w.M, w.N, w.K, w.L, w.TP, w.schedule, w.dtype)
    if w.in_dtype == "e4m3":
        p.set_scales(x.scale_a, x.scale_b)
    for k, v in options.items():
        p.set_option(k, v)
    return p


def _errors_after(w, x, options):
    """Run once through a plan and return (D, timed-out waits)."""
    import torch
    dev = (to_gpu(x.A), to_gpu(x.B), to_gpu(x.C))
    D = empty_out(w)
    with _plan(w, x, options) as p:
        p.run(dev[0], dev[1], dev[2] if w.beta != 0.0 else None, D, w.alpha, w.beta)
        torch.cuda.synchronize()
        n = p.device_errors()
    return D, n


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("sched", SCHEDS)
def test_single_launch_ragged(sched, dtype):
    import torch
    beta = 1.0 if sched.startswith("RS") else 0.5
    w = workloads.small_case(f"fused_{sched}_{dtype}", sched, dtype, 600, 520, 272, 1, 4,
                             1.25, beta, seed=hash((sched, dtype, 7)) % 1000)
    x = workloads.generate(w)
    log("case", w.name, w.M, w.N, w.K, w.TP)
    D, nerr = _errors_after(w, x, FUSED)
    assert nerr == 0
    log("max err", check_full(w, x, D))
    D0 = run_plan(w, x, options={"EXECUTION": 0})
    assert torch.equal(D, D0), "single launch != step launches"


@pytest.mark.parametrize("dtype", ["F32", "BF16_BF16", "E4M3_F32"])
@pytest.mark.parametrize("sched", ["AG_ROT_A", "AG_ROT_B", "RS_TILE_B_ROT_C"])
def test_single_launch_batched(sched, dtype):
    import torch
    w = workloads.small_case(f"fused_batched_{sched}_{dtype}", sched, dtype, 384, 264, 160, 3, 2,
                             0.75, 1.0, seed=23)
    x = workloads.generate(w)
    log("case", w.name)
    D, nerr = _errors_after(w, x, FUSED)
    assert nerr == 0
    check_full(w, x, D)
    assert torch.equal(D, run_plan(w, x, options={"EXECUTION": 0}))


@pytest.mark.parametrize("M,N,K,TP,sched", [
    (8, 16, 16, 8, "AG_ROT_A"),           # one row per step
    (64, 8, 16, 8, "RS_TILE_B_ROT_C"),    # one column per step (2-D chunk copies)
    (16, 24, 48, 8, "AG_ROT_B"),
    (512, 512, 128, 2, "RS_TILE_A_ROT_C"),
    (1024, 256, 64, 16, "AG_ROT_A"),      # more steps than queues
])
@pytest.mark.parametrize("dtype", ["BF16_F32", "E4M3_BF16"])
def test_single_launch_edges(M, N, K, TP, sched, dtype):
    import torch
    w = workloads.small_case(f"fused_edge_{M}x{N}x{K}_{sched}_{dtype}", sched, dtype, M, N, K, 1, TP,
                             1.0, 1.0 if sched.startswith("RS") else 0.0, seed=M + N + K)
    x = workloads.generate(w)
    log("case", w.name)
    D, nerr = _errors_after(w, x, FUSED)
    assert nerr == 0
    check_full(w, x, D)
    assert torch.equal(D, run_plan(w, x, options={"EXECUTION": 0}))


@pytest.mark.parametrize("queues,chunk,group,ahead", [(8, 4096, 2, 2), (1, 4096, 1, 1), (1, 1 << 20, 3, 2),
                                                      (8, 16384, 1, 64), (8, 1 << 28, 7, 1),
                                                      (8, 1 << 21, 1024, 3), (8, 4096, 1, 7),
                                                      (8, 8192, 2, 0), (1, 4096, 1, 0)])
def test_single_launch_queues_chunks_groups(queues, chunk, group, ahead):
    """Work distribution does not change a bit of the result: one queue or
    one per XCD, chunks from 4 KiB (thousands of chunks) to one per shard,
    launch groups from one step to all staged steps, quota-claiming segments
    from none (waiting tiles copy everything) to all."""
    import torch
    for sched in ("AG_ROT_A", "AG_ROT_B", "RS_TILE_B_ROT_C"):
        w = workloads.small_case(f"fused_q{queues}_c{chunk}_g{group}_{sched}", sched, "BF16_F32", 1024,
                                 768, 320, 2, 8, 1.0, 1.0, seed=5)
        x = workloads.generate(w)
        log("case", w.name)
        D, nerr = _errors_after(w, x, {"EXECUTION": 1, "QUEUES": queues, "COPY_CHUNK": chunk,
                                       "STEP_GROUP": group, "COPY_AHEAD": ahead})
        assert nerr == 0
        assert torch.equal(D, run_plan(w, x, options={"EXECUTION": 0})), (queues, chunk, group, ahead,
                                                                          sched)


def test_single_launch_in_place_reduce_scatter():
    """RS with D aliasing C: every chunk's partial is staged before its step's
    tiles overwrite it."""
    import torch
    w = workloads.small_case("fused_inplace", "RS_TILE_A_ROT_C", "BF16_F32", 1024, 512, 256, 1, 4,
                             1.0, 1.0, seed=9)
    x = workloads.generate(w)
    log("case", w.name)
    A, B, C = to_gpu(x.A), to_gpu(x.B), to_gpu(x.C)
    with _plan(w, x, FUSED) as p:
        p.run(A, B, C, C, 1.0, 1.0)
        torch.cuda.synchronize()
        assert p.device_errors() == 0
    check_full(w, x, C)


def test_single_launch_repeated_interleaved_and_concurrent():
    """Counters start from zero on every launch: one plan run repeatedly with
    new operands, two plans interleaved on one stream, and two plans on two
    streams (their launches are ordered by the library)."""
    import torch
    w1 = workloads.small_case("fused_rep_a", "AG_ROT_A", "BF16_F32", 1536, 1024, 512, 1, 4, 1.0, 0.0,
                              seed=31)
    w2 = workloads.small_case("fused_rep_b", "RS_TILE_A_ROT_C", "BF16_F32", 1024, 768, 256, 1, 8, 1.0,
                              1.0, seed=32)
    xs1 = [workloads.generate(workloads.small_case("fused_rep_a", "AG_ROT_A", "BF16_F32", 1536, 1024,
                                                   512, 1, 4, 1.0, 0.0, seed=40 + i)) for i in range(3)]
    x2 = workloads.generate(w2)
    refs1 = [run_plan(w1, x, options={"EXECUTION": 0}) for x in xs1]
    ref2 = run_plan(w2, x2, options={"EXECUTION": 0})
    d1 = [(to_gpu(x.A), to_gpu(x.B)) for x in xs1]
    A2, B2, C2 = to_gpu(x2.A), to_gpu(x2.B), to_gpu(x2.C)
    with _plan(w1, xs1[0], FUSED) as p1, _plan(w2, x2, FUSED) as p2:
        log("case repeated runs")
        for i in range(3):
            D = empty_out(w1)
            p1.run(d1[i][0], d1[i][1], None, D, 1.0, 0.0)
            torch.cuda.synchronize()
            assert torch.equal(D, refs1[i]), f"repeat {i}"
        log("case interleaved plans")
        outs = []
        for i in range(3):
            D1, D2 = empty_out(w1), empty_out(w2)
            p1.run(d1[i][0], d1[i][1], None, D1, 1.0, 0.0)
            p2.run(A2, B2, C2, D2, 1.0, 1.0)
            outs.append((i, D1, D2))
        torch.cuda.synchronize()
        for i, D1, D2 in outs:
            assert torch.equal(D1, refs1[i]) and torch.equal(D2, ref2), f"interleaved {i}"
        log("case two streams")
        s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
        outs = []
        for i in range(3):
            D1, D2 = empty_out(w1), empty_out(w2)
            torch.cuda.synchronize()
            p1.run(d1[i][0], d1[i][1], None, D1, 1.0, 0.0, stream=s1)
            p2.run(A2, B2, C2, D2, 1.0, 1.0, stream=s2)
            outs.append((i, D1, D2))
        torch.cuda.synchronize()
        for i, D1, D2 in outs:
            assert torch.equal(D1, refs1[i]) and torch.equal(D2, ref2), f"two streams {i}"
        assert p1.device_errors() == 0 and p2.device_errors() == 0


def test_single_launch_graph_replay():
    """A single-launch run captured into a HIP graph: every replay (with eager
    work and synchronisation between replays) equals the eager result."""
    import torch
    w = workloads.small_case("fused_graph", "AG_ROT_B", "BF16_BF16", 1024, 1024, 384, 1, 4, 1.0, 0.0,
                             seed=51)
    x = workloads.generate(w)
    ref = run_plan(w, x, options={"EXECUTION": 0})
    A, B = to_gpu(x.A), to_gpu(x.B)
    D = empty_out(w)
    s = torch.cuda.Stream()
    with _plan(w, x, FUSED) as p:
        with torch.cuda.stream(s):
            p.run(A, B, None, D, 1.0, 0.0, stream=s)  # warm-up on the capture stream
        torch.cuda.synchronize()
        assert torch.equal(D, ref)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            p.run(A, B, None, D, 1.0, 0.0, stream=s)
        for i in range(3):
            D.fill_(0)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            log("replay", i)
            assert torch.equal(D, ref), f"replay {i}"
            _ = (A.float() * 2).sum().item()  # eager work between replays
        assert p.device_errors() == 0


def test_single_launch_wait_limit():
    """Failure handling from the host: with a zero wait limit every wait that
    is not already satisfied runs out, is counted, and its workgroup copies
    the strip itself, so both runs are still exact; the counters stay
    consistent, so the next run with the default limit is exact too."""
    import torch
    w = workloads.small_case("fused_limit", "AG_ROT_A", "BF16_F32", 2048, 2048, 1024, 1, 8, 1.0, 0.0,
                             seed=61)
    x = workloads.generate(w)
    ref = run_plan(w, x, options={"EXECUTION": 0})
    A, B = to_gpu(x.A), to_gpu(x.B)
    with _plan(w, x, {"EXECUTION": 1, "WAIT_LIMIT_US": 0}) as p:
        outs = []
        for _ in range(2):
            D = empty_out(w)
            p.run(A, B, None, D, 1.0, 0.0)
            outs.append(D)
        torch.cuda.synchronize()
        n0 = p.device_errors()
        log("timed-out waits with a zero limit:", n0)
        assert n0 > 0
        for i, D in enumerate(outs):
            assert torch.equal(D, ref), f"run {i} that gave up"
        p.set_option("WAIT_LIMIT_US", 1000000)
        D = empty_out(w)
        p.run(A, B, None, D, 1.0, 0.0)
        torch.cuda.synchronize()
        assert p.device_errors() == n0
        assert torch.equal(D, ref)


def test_single_launch_option_errors():
    import communication_tensor_gemm_amd as dg
    with dg.Plan(512, 512, 64, 1, 2, "AG_ROT_A", "BF16_F32") as p:
        for opt, bad in (("EXECUTION", 2), ("QUEUES", 4), ("COPY_CHUNK", 4095), ("COPY_CHUNK", 4104),
                         ("COPY_CHUNK", (1 << 28) + 16), ("WAIT_LIMIT_US", -1), ("COPY_AHEAD", -1),
                         ("COPY_AHEAD", 65)):
            with pytest.raises(dg.DistGemmError):
                p.set_option(opt, bad)
    # plans without staged steps accept the options and run step launches
    with dg.Plan(512, 512, 64, 1, 1, "MONOLITHIC", "BF16_F32") as p:
        p.set_option("EXECUTION", 1)
        p.set_option("COPY_CHUNK", 8192)
        assert p.device_errors() == 0


FULL = ["c2_blog_overlap_f32", "c3_ag_rot_a_bf16_tp8", "c4_rs_tile_a_rot_c_bf16_tp8",
        "c5_ag_rot_b_e4m3_tp8"]


@pytest.mark.parametrize("name", FULL)
def test_single_launch_full_config(name):
    """The full-size workloads in single-launch execution: sampled oracle
    parity, bitwise equality with the monolithic GEMM, no timed-out wait."""
    import torch
    w = workloads.CONFIGS[name]
    log("case", name, "generating inputs")
    x = workloads.generate(w)
    dev = (to_gpu(x.A), to_gpu(x.B), to_gpu(x.C))
    log("case", name, "single-launch run")
    D = empty_out(w)
    with _plan(w, x, FUSED) as p:
        p.run(dev[0], dev[1], dev[2] if w.beta != 0.0 else None, D, w.alpha, w.beta)
        torch.cuda.synchronize()
        assert p.device_errors() == 0
    rows_sched = w.schedule in ("AG_ROT_A", "RS_TILE_A_ROT_C")
    rows = sample_indices(w.M, w.TP if rows_sched else 1, 6, seed=3)
    cols = sample_indices(w.N, 1 if rows_sched else w.TP, 6, seed=4)
    log("case", name, "sampled parity on", len(rows), "x", len(cols))
    log("case", name, "max normalised error", check_sampled(w, x, D, rows, cols))
    Dm = run_plan(w, x, schedule="MONOLITHIC", TP=1, dev=dev)
    assert torch.equal(D, Dm), "single launch != monolithic"
