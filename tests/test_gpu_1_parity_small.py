"""GPU parity at sizes the full oracle handles in seconds: every schedule and
element type, shapes spanning several 256 x 256 tiles with ragged M, N and K
tails, batches, and the degenerate cases.  Every call goes through the C ABI;
every output element is compared with the fp64 oracle."""
import numpy as np
import pytest

import workloads
from gpu_helpers import check_full, log, run_plan, to_gpu

pytestmark = pytest.mark.gpu

SCHEDS = ["AG_ROT_A", "AG_ROT_B", "RS_TILE_A_ROT_C", "RS_TILE_B_ROT_C", "MONOLITHIC"]
DTYPES = ["F32", "BF16_F32", "BF16_BF16", "E4M3_BF16", "E4M3_F32"]


def test_c1_tiny_rotating_a_f32():
    w = workloads.CONFIGS["c1_tiny_ag_rot_a_f32"]
    x = workloads.generate(w)
    log("case c1", w)
    D = run_plan(w, x)
    err = check_full(w, x, D)
    log("c1 max normalised error", err)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("sched", SCHEDS)
def test_grid_ragged(sched, dtype):
    # 600 x 520 with TP=4: 150-row / 130-column steps, 3 x 3 tiles monolithic;
    # K = 272 leaves a partial K tile for every element type.
    beta = 1.0 if sched.startswith("RS") else 0.5
    w = workloads.small_case(f"grid_{sched}_{dtype}", sched, dtype, 600, 520, 272, 1, 4,
                             1.25, beta, seed=hash((sched, dtype)) % 1000)
    x = workloads.generate(w)
    log("case", w.name, w.M, w.N, w.K, w.TP)
    D = run_plan(w, x)
    log("max err", check_full(w, x, D))


@pytest.mark.parametrize("dtype", ["F32", "BF16_BF16", "E4M3_F32"])
@pytest.mark.parametrize("sched", ["AG_ROT_A", "RS_TILE_B_ROT_C"])
def test_batched(sched, dtype):
    w = workloads.small_case(f"batched_{sched}_{dtype}", sched, dtype, 384, 264, 160, 3, 2,
                             0.75, 1.0, seed=17)
    x = workloads.generate(w)
    log("case", w.name)
    D = run_plan(w, x)
    check_full(w, x, D)


@pytest.mark.parametrize("M,N,K,TP,sched", [
    (1, 1, 16, 1, "MONOLITHIC"),          # single element, one partial K tile
    (1, 300, 16, 1, "AG_ROT_B"),
    (300, 1, 48, 1, "RS_TILE_A_ROT_C"),
    (8, 16, 16, 8, "AG_ROT_A"),           # one row per step
    (64, 8, 16, 8, "RS_TILE_B_ROT_C"),    # one column per step
    (257, 255, 1040, 1, "MONOLITHIC"),    # one past / one short of a tile
    (512, 512, 128, 2, "AG_ROT_B"),       # exact tiles, exact K tiles
])
@pytest.mark.parametrize("dtype", ["BF16_F32", "E4M3_BF16"])
def test_edge_shapes(M, N, K, TP, sched, dtype):
    w = workloads.small_case(f"edge_{M}_{N}_{K}", sched, dtype, M, N, K, 1, TP, 1.0,
                             1.0 if sched.startswith("RS") else 0.0, seed=M + N + K)
    x = workloads.generate(w)
    log("case", w.name, sched, dtype)
    D = run_plan(w, x)
    check_full(w, x, D)


@pytest.mark.parametrize("execution", [0, 1])
@pytest.mark.parametrize("group", [2, 3, 8])
@pytest.mark.parametrize("dtype", ["F32", "BF16_BF16", "E4M3_F32"])
@pytest.mark.parametrize("sched", ["AG_ROT_A", "AG_ROT_B", "RS_TILE_A_ROT_C", "RS_TILE_B_ROT_C"])
def test_step_groups(sched, dtype, group, execution):
    # TP=8 on 600 x 520: 75-row / 65-column shards, so merged launches have
    # tiles that straddle shard boundaries; L=2 exercises the batch strides
    # of the side-by-side staging layout.
    import torch
    beta = 1.0 if sched.startswith("RS") else 0.5
    w = workloads.small_case(f"group_{sched}_{dtype}_{group}", sched, dtype, 600, 520, 96, 2, 8,
                             1.5, beta, seed=group * 7 + len(sched))
    x = workloads.generate(w)
    log("case", w.name, "STEP_GROUP", group, "EXECUTION", execution)
    dev = (to_gpu(x.A), to_gpu(x.B), to_gpu(x.C))
    Dg = run_plan(w, x, dev=dev, options={"STEP_GROUP": group, "EXECUTION": execution})
    check_full(w, x, Dg)
    D1 = run_plan(w, x, dev=dev, options={"STEP_GROUP": 1, "EXECUTION": execution})
    assert torch.equal(Dg, D1), "grouped launches differ from one launch per step"


@pytest.mark.parametrize("dtype", ["F32", "BF16_BF16", "E4M3_BF16"])
@pytest.mark.parametrize("sched", ["AG_ROT_A", "AG_ROT_B", "RS_TILE_A_ROT_C", "RS_TILE_B_ROT_C"])
def test_copy_engines_agree(sched, dtype):
    # 600 x 518 at TP=2 with L=2: odd row and column widths, so the library
    # copy kernel takes its 16-, 4- and 1-byte paths; every engine must give
    # the same bits
    import torch
    beta = 1.0 if sched.startswith("RS") else 0.25
    w = workloads.small_case(f"engines_{sched}_{dtype}", sched, dtype, 600, 518, 112, 2, 2, 1.0,
                             beta, seed=5 + len(sched))
    x = workloads.generate(w)
    dev = (to_gpu(x.A), to_gpu(x.B), to_gpu(x.C))
    log("case", w.name)
    outs = [run_plan(w, x, dev=dev, options={"COPY_ENGINE": e, "EXECUTION": 0}) for e in (0, 1, 2)]
    check_full(w, x, outs[2])
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[1], outs[2])
    # the single launch's own chunked copy (16-, 4- and 1-byte units alike)
    assert torch.equal(outs[2], run_plan(w, x, dev=dev, options={"EXECUTION": 1}))


def test_alpha_zero_and_beta_zero_ignores_c():
    import torch
    w = workloads.small_case("a0", "AG_ROT_A", "BF16_F32", 512, 256, 64, 1, 2, 0.0, 0.75, seed=3)
    x = workloads.generate(w, need_c=True)
    D = run_plan(w, x)
    expect = 0.75 * x.C.astype(np.float64)
    assert np.array_equal(D.cpu().numpy().astype(np.float64), expect.astype(np.float32))
    # beta = 0: C is not read even when it holds NaN
    import communication_tensor_gemm_amd as dg
    A, B = to_gpu(x.A), to_gpu(x.B)
    Cnan = torch.full((1, 512, 256), float("nan"), device="cuda")
    D0 = torch.empty((1, 512, 256), device="cuda")
    w0 = workloads.small_case("b0", "AG_ROT_A", "BF16_F32", 512, 256, 64, 1, 2, 1.0, 0.0, seed=3)
    with dg.Plan(512, 256, 64, 1, 2, "AG_ROT_A", "BF16_F32") as p:
        p.run(A, B, Cnan, D0, 1.0, 0.0)
        torch.cuda.synchronize()
    assert torch.isfinite(D0).all()
    check_full(w0, x, D0)


@pytest.mark.parametrize("sched", ["RS_TILE_A_ROT_C", "RS_TILE_B_ROT_C", "AG_ROT_A"])
def test_d_aliases_c(sched):
    w = workloads.small_case("alias", sched, "BF16_F32", 512, 384, 96, 1, 4, 1.0, 1.0, seed=5)
    x = workloads.generate(w)
    A, B, C = to_gpu(x.A), to_gpu(x.B), to_gpu(x.C)
    D = run_plan(w, x, dev=(A, B, C), out=C)     # D is C
    check_full(w, x, D)


def test_run_errors():
    import torch
    import communication_tensor_gemm_amd as dg
    A = torch.zeros(64 * 64, dtype=torch.int16, device="cuda")
    D = torch.zeros(64 * 64, dtype=torch.float32, device="cuda")
    with dg.Plan(64, 64, 64, 1, 2, "RS_TILE_A_ROT_C", "BF16_F32") as p:
        with pytest.raises(dg.DistGemmError) as ei:
            dg.dist_gemm_run(p.handle, A, A, None, D, 1.0, 1.0)   # beta != 0 without C
        assert ei.value.status == -1
        with pytest.raises(dg.DistGemmError):
            dg.dist_gemm_run(p.handle, A, A, D, D, float("nan"), 1.0)
        with pytest.raises(dg.DistGemmError):
            dg.dist_gemm_set_option(p.handle, "COMPUTE_STREAMS", 3)
        for bad in (0, 9):
            with pytest.raises(dg.DistGemmError):
                dg.dist_gemm_set_option(p.handle, "COPY_STREAMS", bad)
        for bad in (0, 1025):
            with pytest.raises(dg.DistGemmError):
                dg.dist_gemm_set_option(p.handle, "STEP_GROUP", bad)
        for bad in (-1, 3):
            with pytest.raises(dg.DistGemmError):
                dg.dist_gemm_set_option(p.handle, "COPY_ENGINE", bad)
        with pytest.raises(ValueError):
            p.run(A[:10], A, D, D, 1.0, 1.0)               # too small for 64 x 64
    with pytest.raises(dg.DistGemmError) as ei:
        dg.Plan(64, 64, 60, 1, 2, "AG_ROT_A", "BF16_F32")
    assert ei.value.status == -2
