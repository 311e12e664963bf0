"""GPU tests of dist_gemm_run_noalloc, the entry point that allocates nothing
(its gathered image, tables and counters live in a file-scope device array).

Every call goes through the C ABI and is compared bit for bit with the
plan-based dist_gemm_run of the same problem and operands (the default
single-launch execution, the same kernels), and with the fp64 oracle.  Calls
come two in a row, the second on a smaller problem, so the second finds the
array holding the first call's tables, counters and gathered shards.
"""
import numpy as np
import pytest

import workloads
from gpu_helpers import check_full, empty_out, log, run_plan, to_gpu

pytestmark = pytest.mark.gpu


def _noalloc(w, x, dev, stream=None):
    import torch
    import communication_tensor_gemm_amd as dg
    A, B, C = dev
    D = empty_out(w)
    dg.dist_gemm_run_noalloc(w.M, w.N, w.K, w.L, w.TP, w.schedule, w.dtype, A, B,
                             C if w.beta != 0.0 else None, D, w.alpha, w.beta, x.scale_a, x.scale_b,
                             stream)
    if stream is None:
        torch.cuda.synchronize()
    return D


CASES = [
    # (schedule, dtype, first (M, N, K, L, TP), second, smaller)
    ("AG_ROT_A", "BF16_F32", (1024, 768, 512, 2, 8), (600, 520, 272, 1, 4)),
    ("AG_ROT_B", "E4M3_BF16", (768, 3328, 256, 1, 8), (256, 520, 128, 2, 4)),
    ("RS_TILE_A_ROT_C", "BF16_F32", (2048, 1024, 256, 1, 8), (520, 384, 64, 1, 2)),
    ("RS_TILE_B_ROT_C", "F32", (512, 2048, 128, 1, 4), (384, 264, 32, 2, 2)),
    ("MONOLITHIC", "BF16_BF16", (512, 512, 256, 1, 1), (256, 128, 64, 1, 1)),
]


@pytest.mark.parametrize("sched,dtype,big,small", CASES)
def test_noalloc_two_calls_match_plan_run(sched, dtype, big, small):
    import torch
    for k, (M, N, K, L, TP) in enumerate((big, small)):
        beta = 1.0 if sched.startswith("RS") else (0.5 if k == 0 else 0.0)
        w = workloads.small_case(f"noalloc_{sched}_{dtype}_{k}", sched, dtype, M, N, K, L, TP, 1.25, beta,
                                 seed=300 + 7 * k)
        x = workloads.generate(w)
        log("case", w.name, (M, N, K, L, TP))
        dev = (to_gpu(x.A), to_gpu(x.B), to_gpu(x.C))
        D = _noalloc(w, x, dev)
        ref = run_plan(w, x, dev=dev, options={"EXECUTION": 1})
        assert torch.equal(D, ref), f"no-alloc call {k} != plan run"
        check_full(w, x, D)


def test_noalloc_reduce_scatter_in_place_and_beta_zero():
    import torch
    import communication_tensor_gemm_amd as dg
    w = workloads.small_case("noalloc_rs_inplace", "RS_TILE_A_ROT_C", "BF16_F32", 1024, 512, 256, 1, 4, 1.0,
                             1.0, seed=311)
    x = workloads.generate(w)
    A, B, C = to_gpu(x.A), to_gpu(x.B), to_gpu(x.C)
    dg.dist_gemm_run_noalloc(w.M, w.N, w.K, w.L, w.TP, w.schedule, w.dtype, A, B, C, C, 1.0, 1.0, 1.0, 1.0)
    torch.cuda.synchronize()
    check_full(w, x, C)
    w0 = workloads.small_case("noalloc_rs_b0", "RS_TILE_B_ROT_C", "BF16_F32", 512, 1024, 128, 1, 4, 1.0, 0.0,
                              seed=312)
    x0 = workloads.generate(w0)
    D = _noalloc(w0, x0, (to_gpu(x0.A), to_gpu(x0.B), None))
    check_full(w0, x0, D)


def test_noalloc_graph_capture_replays():
    """A captured call (the use it is for): every replay, with eager work and
    other no-alloc calls between the replays, equals the eager call."""
    import torch
    import communication_tensor_gemm_amd as dg
    w = workloads.small_case("noalloc_graph", "AG_ROT_A", "BF16_F32", 1024, 1024, 384, 1, 8, 1.0, 0.0,
                             seed=321)
    x = workloads.generate(w)
    dev = (to_gpu(x.A), to_gpu(x.B), None)
    ref = _noalloc(w, x, dev)
    other = workloads.small_case("noalloc_graph_other", "AG_ROT_B", "BF16_F32", 512, 768, 128, 1, 4, 1.0, 0.0,
                                 seed=322)
    xo = workloads.generate(other)
    devo = (to_gpu(xo.A), to_gpu(xo.B), None)
    s = torch.cuda.Stream()
    D = empty_out(w)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        dg.dist_gemm_run_noalloc(w.M, w.N, w.K, w.L, w.TP, w.schedule, w.dtype, dev[0], dev[1], None, D,
                                 1.0, 0.0, 1.0, 1.0, s)
    for i in range(3):
        D.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(D, ref), f"replay {i}"
        _noalloc(other, xo, devo)  # another call rewrites the array between replays
        _ = (dev[0].float() * 2).sum().item()


def test_noalloc_limits_and_errors():
    """Rejected before any device work: the calls below never touch memory."""
    import torch
    import communication_tensor_gemm_amd as dg
    A, B, D = (torch.zeros(16, dtype=torch.int16, device="cuda") for _ in range(3))
    # a gathered A of 8192 x 4096 bf16 (64 MiB) exceeds the 32 MiB array
    with pytest.raises(dg.DistGemmError) as ei:
        dg.dist_gemm_run_noalloc(8192, 256, 4096, 1, 8, "AG_ROT_A", "BF16_F32", A, B, None, D, 1.0, 0.0, 1.0, 1.0)
    assert ei.value.status == -3
    assert b"32 MiB" in dg.lib.dist_gemm_last_error(None)
    # 32 steps
    with pytest.raises(dg.DistGemmError) as ei:
        dg.dist_gemm_run_noalloc(512, 256, 64, 1, 32, "AG_ROT_A", "BF16_F32", A, B, None, D, 1.0, 0.0, 1.0, 1.0)
    assert ei.value.status == -3
    # a missing operand, an indivisible shape, D aliasing A
    for args, status in (((512, 256, 64, 1, 4, "AG_ROT_A", "BF16_F32", A, None, None, D), -1),
                         ((510, 256, 64, 1, 4, "AG_ROT_A", "BF16_F32", A, B, None, D), -2),
                         ((512, 256, 64, 1, 4, "AG_ROT_A", "BF16_F32", A, B, None, A), -1)):
        with pytest.raises(dg.DistGemmError) as ei:
            dg.dist_gemm_run_noalloc(*args, 1.0, 0.0, 1.0, 1.0)
        assert ei.value.status == status
