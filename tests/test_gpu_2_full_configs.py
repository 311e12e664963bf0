"""GPU parity at the four full-size workloads, in the launch configuration the
benchmark times (the library defaults: one persistent launch per run).

The oracle computes sampled outputs one by one: rows and columns that cover
every step block, both sides of 256-tile edges, and random positions.  The
properties that hold at any size are checked on the whole output, bitwise:
the schedule equals the monolithic GEMM of the same kernel, and the
step-launch execution with every copy engine, copy-stream count, compute
stream count and step grouping equals it too.
"""
import numpy as np
import pytest

import workloads
from gpu_helpers import check_sampled, log, run_plan, sample_indices, to_gpu

pytestmark = pytest.mark.gpu

FULL = ["c2_blog_overlap_f32", "c3_ag_rot_a_bf16_tp8", "c4_rs_tile_a_rot_c_bf16_tp8",
        "c5_ag_rot_b_e4m3_tp8"]


@pytest.mark.parametrize("name", FULL)
def test_full_config(name):
    import torch
    w = workloads.CONFIGS[name]
    log("case", name, "generating inputs")
    x = workloads.generate(w)
    dev = (to_gpu(x.A), to_gpu(x.B), to_gpu(x.C))
    log("case", name, "run schedule", w.schedule, "TP", w.TP)
    D = run_plan(w, x, dev=dev)
    rows_sched = w.schedule in ("AG_ROT_A", "RS_TILE_A_ROT_C")
    rows = sample_indices(w.M, w.TP if rows_sched else 1, 6, seed=1)
    cols = sample_indices(w.N, 1 if rows_sched else w.TP, 6, seed=2)
    log("case", name, "sampled parity on", len(rows), "x", len(cols))
    err = check_sampled(w, x, D, rows, cols)
    log("case", name, "max normalised error", err)

    log("case", name, "bitwise invariants")
    Dm = run_plan(w, x, schedule="MONOLITHIC", TP=1, dev=dev)
    assert torch.equal(D, Dm), "schedule != monolithic"
    del Dm
    # step-launch execution and its options
    D1 = run_plan(w, x, dev=dev, options={"EXECUTION": 0, "COMPUTE_STREAMS": 1})
    assert torch.equal(D, D1), "step launches on one compute stream != the default"
    del D1
    for e in (0, 1, 2):
        Db = run_plan(w, x, dev=dev, options={"EXECUTION": 0, "COPY_ENGINE": e})
        assert torch.equal(D, Db), f"step launches with copy engine {e} != the default"
        del Db
    for n in (1, 7):
        Dn = run_plan(w, x, dev=dev, options={"EXECUTION": 0, "COPY_STREAMS": n})
        assert torch.equal(D, Dn), f"step launches with {n} copy streams != the default"
        del Dn
    for g in (1, 2, 7):
        for ex in (0, 1):
            Dg = run_plan(w, x, dev=dev, options={"EXECUTION": ex, "STEP_GROUP": g})
            assert torch.equal(D, Dg), f"execution {ex}, step groups of {g} != the default"
            del Dg
    if w.out_dtype == "f32":
        assert torch.isfinite(D).all()
    torch.cuda.synchronize()
