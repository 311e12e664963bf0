"""The step timeline (DIST_GEMM_OPT_STEP_TIMING), and the whole schedule
captured into a HIP graph and replayed.  Every call goes through the C ABI."""
import numpy as np
import pytest

import workloads
from gpu_helpers import check_full, empty_out, log, to_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("sched", ["AG_ROT_A", "RS_TILE_B_ROT_C"])
@pytest.mark.parametrize("group", [1, 2])
def test_step_timeline(sched, group):
    import torch
    import communication_tensor_gemm_amd as dg
    beta = 1.0 if sched.startswith("RS") else 0.0
    w = workloads.small_case(f"tl_{sched}", sched, "BF16_F32", 1024, 1024, 256, 1, 8, 1.0, beta,
                             seed=11)
    x = workloads.generate(w)
    A, B, C = to_gpu(x.A), to_gpu(x.B), to_gpu(x.C)
    D = empty_out(w)
    log("case timeline", sched, "group", group)
    with dg.Plan(w.M, w.N, w.K, w.L, w.TP, sched, w.dtype) as p:
        p.set_option("EXECUTION", 0)
        p.set_option("STEP_GROUP", group)
        with pytest.raises(dg.DistGemmError):
            p.step_timeline()                       # nothing recorded yet
        p.set_option("STEP_TIMING", 3)
        for _ in range(4):
            p.run(A, B, C if beta else None, D, w.alpha, beta)
        torch.cuda.synchronize()
        tl = p.step_timeline()
        st = p.steps()
        times = p.step_times()
    check_full(w, x, D)
    assert len(tl) == w.TP and len(times) == 3 * w.TP
    for (copy, b, e), s in zip(tl, st):
        assert 0.0 <= b <= e
        staged = s[2]
        if staged:
            # the launch waits for its copy (event timestamps of different
            # streams can be a few tens of microseconds apart)
            assert copy >= 0.0 and copy <= b + 0.1
        else:
            assert copy == -1.0
    launches = sorted({(b, e) for _, b, e in tl})
    # group 2 at TP=8: {0}, {1,2}, {3,4}, {5,6}, {7} for both schedules (for the
    # reduce-scatter order the last step wraps to shard 0 and launches alone)
    expect = w.TP if group == 1 else 5
    assert len(launches) == expect
    assert all(t > 0 for t in times)


def test_single_launch_timeline():
    """A single-launch run reports the device's own stamps per step: the last
    strip of a staged step complete, and the first and last tile of the step.
    Here (1024 columns over 8 steps) every 256-column strip straddles two
    shards and belongs to the later one, so the even steps have no strip and
    report -1; the odd steps report copies, then tiles, inside the launch."""
    import torch
    import communication_tensor_gemm_amd as dg
    w = workloads.small_case("tl_single", "AG_ROT_B", "BF16_F32", 1024, 1024, 256, 1, 8, 1.0, 0.0,
                             seed=12)
    x = workloads.generate(w)
    A, B = to_gpu(x.A), to_gpu(x.B)
    D = empty_out(w)
    with dg.Plan(w.M, w.N, w.K, w.L, w.TP, w.schedule, w.dtype) as p:
        p.set_option("EXECUTION", 1)
        p.set_option("STEP_TIMING", 2)
        for _ in range(3):
            p.run(A, B, None, D, 1.0, 0.0)
        torch.cuda.synchronize()
        tl = p.step_timeline()
        times = p.step_times()
    check_full(w, x, D)
    log("timeline", tl)
    assert [s for s, (_, b, _) in enumerate(tl) if b >= 0] == [1, 3, 5, 7]
    for s, (c, b, e) in enumerate(tl):
        if s % 2 == 0:
            assert (c, b, e) == (-1.0, -1.0, -1.0)
        else:
            # a strip's tiles start only once it is complete; the step's last
            # strip may complete after its first tile began (tile-granular)
            assert 0.0 <= c <= e and 0.0 <= b <= e
    assert len(times) == 2 * w.TP and all(t > 0 for t in times)


@pytest.mark.parametrize("execution", [0, 1])
@pytest.mark.parametrize("sched,dtype", [("AG_ROT_A", "BF16_F32"), ("RS_TILE_A_ROT_C", "BF16_F32"),
                                         ("AG_ROT_B", "E4M3_BF16")])
def test_graph_capture_replay(sched, dtype, execution):
    """The run is capturable: one capture of dist_gemm_run on a side stream,
    replayed three times with eager work between the replays; every replay
    equals the eager run bit for bit."""
    import torch
    import communication_tensor_gemm_amd as dg
    beta = 1.0 if sched.startswith("RS") else 0.0
    w = workloads.small_case(f"graph_{sched}", sched, dtype, 768, 1024, 384, 1, 4, 1.0, beta,
                             seed=21)
    x = workloads.generate(w)
    A, B, C = to_gpu(x.A), to_gpu(x.B), to_gpu(x.C)
    D_eager = empty_out(w)
    D_graph = empty_out(w)
    log("case graph capture", sched, dtype)
    with dg.Plan(w.M, w.N, w.K, w.L, w.TP, sched, w.dtype) as p:
        if w.in_dtype == "e4m3":
            p.set_scales(x.scale_a, x.scale_b)
        p.set_option("EXECUTION", execution)
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            p.run(A, B, C if beta else None, D_eager, w.alpha, beta, stream=s.cuda_stream)
        s.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            p.run(A, B, C if beta else None, D_graph, w.alpha, beta, stream=s.cuda_stream)
        for rep in range(3):
            D_graph.fill_(-7)                         # eager work between replays
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            log("replay", rep)
            assert torch.equal(D_graph, D_eager), f"replay {rep} differs from the eager run"
        del g
    check_full(w, x, D_eager)
