"""GPU tests of the scaled matmul's fp8 output (dtype E4M3_E4M3): the result
scale (dist_gemm_set_result_scale) multiplies the fp32 result before the
cast to e4m3fn, which rounds to nearest even and saturates at +-448; the
fast-accumulate option changes nothing on gfx950.

Every case is checked against the fp64 oracle (result scale applied before
its one rounding; the parity metric clips to +-448 and allows half a
spacing of three mantissa bits) and bit for bit against the monolithic GEMM
with the same result scale.
"""
import numpy as np
import pytest

import workloads
from gpu_helpers import check_full, empty_out, log, run_plan, to_gpu

pytestmark = pytest.mark.gpu

SCHEDS = ["AG_ROT_A", "AG_ROT_B", "RS_TILE_A_ROT_C", "RS_TILE_B_ROT_C"]


@pytest.mark.parametrize("execution", [1, 0])
@pytest.mark.parametrize("sched", SCHEDS)
def test_fp8_output_with_result_scale(sched, execution):
    import torch
    beta = 1.0 if sched.startswith("RS") else 0.5
    for (M, N, K, L, TP), s in (((600, 520, 272, 1, 4), 0.25), ((512, 768, 128, 2, 8), 3.0)):
        w = workloads.small_case(f"fp8out_{sched}_{M}", sched, "E4M3_E4M3", M, N, K, L, TP, 1.25, beta,
                                 seed=M + N)
        x = workloads.generate(w)
        log("case", w.name, "execution", execution, "result scale", s)
        D = run_plan(w, x, options={"EXECUTION": execution}, result_scale=s)
        check_full(w, x, D, result_scale=s)
        assert torch.equal(D, run_plan(w, x, schedule="MONOLITHIC", TP=1, result_scale=s))


def test_fp8_output_saturates():
    """A result scale that drives most results past 448: they come out as
    exactly +-448 (0x7E / 0xFE), the rest rounded."""
    import torch
    w = workloads.small_case("fp8out_sat", "AG_ROT_B", "E4M3_E4M3", 512, 512, 256, 1, 4, 1.0, 0.0, seed=17)
    x = workloads.generate(w)
    D = run_plan(w, x, options={"EXECUTION": 1}, result_scale=300.0)
    check_full(w, x, D, result_scale=300.0)
    codes = D.view(torch.uint8).cpu().numpy() & 0x7F
    assert (codes == 0x7E).mean() > 0.5 and not np.any(codes == 0x7F)


def test_fp8_output_bias_and_in_place_reduce_scatter():
    import torch
    import communication_tensor_gemm_amd as dg
    w = workloads.small_case("fp8out_rs_inplace", "RS_TILE_A_ROT_C", "E4M3_E4M3", 1024, 520, 256, 1, 4,
                             1.0, 1.0, seed=19)
    x = workloads.generate(w)
    g = np.random.default_rng(3)
    bias = torch.from_numpy(np.ascontiguousarray(
        torch.from_numpy(g.standard_normal(w.N).astype(np.float32)).to(torch.float8_e4m3fn)
        .view(torch.uint8).numpy())).cuda()
    A, B, C = to_gpu(x.A), to_gpu(x.B), to_gpu(x.C)
    with dg.Plan(w.M, w.N, w.K, w.L, w.TP, w.schedule, w.dtype) as p:
        p.set_scales(x.scale_a, x.scale_b)
        p.set_result_scale(0.5)
        p.set_bias(bias)
        p.run(A, B, C, C, 1.0, 1.0)
        torch.cuda.synchronize()
    check_full(w, x, C, bias=bias.cpu().numpy(), result_scale=0.5)


@pytest.mark.parametrize("dtype", ["E4M3_BF16", "E4M3_E4M3", "BF16_F32"])
def test_fast_accumulate_changes_nothing(dtype):
    import torch
    w = workloads.small_case(f"fastacc_{dtype}", "AG_ROT_A", dtype, 768, 520, 512, 1, 4, 1.0, 0.0, seed=23)
    x = workloads.generate(w)
    for execution in (1, 0):
        D0 = run_plan(w, x, options={"EXECUTION": execution, "FAST_ACCUM": 0})
        D1 = run_plan(w, x, options={"EXECUTION": execution, "FAST_ACCUM": 1})
        assert torch.equal(D0, D1)
    check_full(w, x, D1)


def test_result_scale_errors():
    import communication_tensor_gemm_amd as dg
    with dg.Plan(256, 256, 64, 1, 2, "AG_ROT_A", "BF16_F32") as p:
        p.set_result_scale(1.0)                  # the identity is accepted on any output
        with pytest.raises(dg.DistGemmError) as ei:
            p.set_result_scale(2.0)
        assert ei.value.status == -3
        with pytest.raises(dg.DistGemmError):
            p.set_option("FAST_ACCUM", 2)
    with dg.Plan(256, 256, 64, 1, 2, "AG_ROT_A", "E4M3_E4M3") as p:
        with pytest.raises(dg.DistGemmError) as ei:
            p.set_result_scale(float("inf"))
        assert ei.value.status == -1
