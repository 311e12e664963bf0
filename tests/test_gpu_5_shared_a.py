"""GPU tests of DIST_GEMM_OPT_SHARED_A: one A (M x K) multiplied by each of L
Bs, with one output per B -- the several-B form of the fused all-gather
matmul on the PyTorch symmetric-memory page (one gathered A shared by, e.g.,
the gate and up projections).

The oracle sees the same A repeated for every batch; the GPU gets one copy
of it.  Every schedule, both executions, full oracle parity and bitwise
equality with the L products run one by one as separate plans.
"""
import dataclasses

import numpy as np
import pytest

import workloads
from gpu_helpers import check_full, empty_out, log, to_gpu

pytestmark = pytest.mark.gpu


def _shared_inputs(w):
    x = workloads.generate(w)
    A1 = np.ascontiguousarray(x.A[:1])
    return dataclasses.replace(x, A=np.ascontiguousarray(np.broadcast_to(A1, x.A.shape))), A1


@pytest.mark.parametrize("execution", [0, 1])
@pytest.mark.parametrize("dtype", ["BF16_F32", "E4M3_BF16", "F32"])
@pytest.mark.parametrize("sched", ["AG_ROT_A", "AG_ROT_B", "RS_TILE_A_ROT_C", "RS_TILE_B_ROT_C",
                                   "MONOLITHIC"])
def test_shared_a(sched, dtype, execution):
    import torch
    import communication_tensor_gemm_amd as dg
    TP = 1 if sched == "MONOLITHIC" else 4
    beta = 1.0 if sched.startswith("RS") else 0.5
    w = workloads.small_case(f"shared_{sched}_{dtype}", sched, dtype, 640, 520, 272, 3, TP, 1.25,
                             beta, seed=hash((sched, dtype)) % 997)
    x, A1 = _shared_inputs(w)
    log("case", w.name, "execution", execution)
    A, B, C = to_gpu(A1), to_gpu(x.B), to_gpu(x.C)
    D = empty_out(w)
    with dg.Plan(w.M, w.N, w.K, w.L, w.TP, sched, w.dtype) as p:
        if w.in_dtype == "e4m3":
            p.set_scales(x.scale_a, x.scale_b)
        p.set_option("EXECUTION", execution)
        p.set_option("SHARED_A", 1)
        p.run(A, B, C, D, w.alpha, w.beta)
        torch.cuda.synchronize()
        assert p.device_errors() == 0
    check_full(w, x, D)
    # the same products one at a time, each a plan of its own
    for l in range(w.L):
        Dl = empty_out(dataclasses.replace(w, L=1))
        with dg.Plan(w.M, w.N, w.K, 1, w.TP, sched, w.dtype) as p:
            if w.in_dtype == "e4m3":
                p.set_scales(x.scale_a, x.scale_b)
            p.set_option("EXECUTION", execution)
            p.run(A, B[l], C[l], Dl, w.alpha, w.beta)
            torch.cuda.synchronize()
        assert torch.equal(D[l], Dl[0]), f"batch {l} != its own run"


def test_shared_a_toggle_and_sizes():
    """Switching the option back and forth on one plan keeps both layouts
    exact, and the binding checks A against the layout in force."""
    import torch
    import communication_tensor_gemm_amd as dg
    w = workloads.small_case("shared_toggle", "AG_ROT_A", "BF16_F32", 1024, 512, 128, 2, 4, 1.0, 0.0,
                             seed=77)
    x, A1 = _shared_inputs(w)
    A_full, A_one, B = to_gpu(x.A), to_gpu(A1), to_gpu(x.B)
    with dg.Plan(w.M, w.N, w.K, w.L, w.TP, w.schedule, w.dtype) as p:
        for shared in (1, 0, 1):
            p.set_option("SHARED_A", shared)
            D = empty_out(w)
            p.run(A_one if shared else A_full, B, None, D, 1.0, 0.0)
            torch.cuda.synchronize()
            check_full(w, x, D)
        with pytest.raises(ValueError):
            p.set_option("SHARED_A", 0)
            p.run(A_one, B, None, empty_out(w), 1.0, 0.0)   # one batch of A, L = 2 needed
        with pytest.raises(dg.DistGemmError):
            p.set_option("SHARED_A", 2)
