"""GPU tests of the scaled-matmul bias (dist_gemm_set_bias): D = alpha*sa*sb*A*B
+ beta*C + bias[j], with the bias in the output element type.  Every schedule
and element type, both executions, against the fp64 oracle (which adds the
same decoded bias); an unaligned bias takes the element-wise epilogue; the
bias can be removed again.
"""
import numpy as np
import pytest

import workloads
from gpu_helpers import check_full, empty_out, log, to_gpu

pytestmark = pytest.mark.gpu

SCHEDS = ["AG_ROT_A", "AG_ROT_B", "RS_TILE_A_ROT_C", "RS_TILE_B_ROT_C", "MONOLITHIC"]


def _bias_bytes(N, out_elem, seed, scale=0.5):
    import torch
    v = (np.random.default_rng(seed).standard_normal(N) * scale).astype(np.float32)
    if out_elem == "f32":
        return v
    return torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _run(w, x, bias_dev, execution, D=None):
    import torch
    import communication_tensor_gemm_amd as dg
    A, B, C = to_gpu(x.A), to_gpu(x.B), to_gpu(x.C)
    D = empty_out(w) if D is None else D
    with dg.Plan(w.M, w.N, w.K, w.L, w.TP, w.schedule, w.dtype) as p:
        if w.in_dtype == "e4m3":
            p.set_scales(x.scale_a, x.scale_b)
        p.set_option("EXECUTION", execution)
        p.set_bias(bias_dev)
        p.run(A, B, C if w.beta != 0 else None, D, w.alpha, w.beta)
        torch.cuda.synchronize()
        assert p.device_errors() == 0
    return D


@pytest.mark.parametrize("execution", [0, 1])
@pytest.mark.parametrize("dtype", ["F32", "BF16_F32", "BF16_BF16", "E4M3_BF16", "E4M3_F32"])
@pytest.mark.parametrize("sched", SCHEDS)
def test_bias(sched, dtype, execution):
    TP = 1 if sched == "MONOLITHIC" else 4
    beta = 1.0 if sched.startswith("RS") else 0.5
    w = workloads.small_case(f"bias_{sched}_{dtype}", sched, dtype, 600, 520, 272, 2, TP, 1.25, beta,
                             seed=hash((sched, dtype, 3)) % 991)
    x = workloads.generate(w)
    bias = _bias_bytes(w.N, w.out_dtype, seed=len(sched) + len(dtype))
    log("case", w.name, "execution", execution)
    D = _run(w, x, to_gpu(bias), execution)
    log("max err", check_full(w, x, D, bias=bias))


@pytest.mark.parametrize("dtype", ["BF16_F32", "E4M3_BF16"])
def test_bias_unaligned_and_removed(dtype):
    """A bias one element past a 16-byte boundary (the fp32 epilogue then
    stores element by element), and set_bias(None) giving the plain result."""
    import torch
    w = workloads.small_case(f"bias_unaligned_{dtype}", "AG_ROT_A", dtype, 512, 768, 256, 1, 2, 1.0, 0.0,
                             seed=8)
    x = workloads.generate(w)
    bias = _bias_bytes(w.N, w.out_dtype, seed=2)
    store = to_gpu(np.concatenate([bias[:1], bias]))
    D = _run(w, x, store[1:], 1)
    check_full(w, x, D, bias=bias)
    D0 = _run(w, x, None, 1)
    check_full(w, x, D0)
    assert not torch.equal(D, D0)


def test_bias_full_c3_sampled():
    """The c3 workload with a bias: sampled oracle parity; the bias-free part
    is bitwise the run without bias plus the bias (fp32 output, one rounding)."""
    import torch
    from gpu_helpers import check_sampled, sample_indices
    w = workloads.CONFIGS["c3_ag_rot_a_bf16_tp8"]
    x = workloads.generate(w)
    bias = _bias_bytes(w.N, "f32", seed=5)
    D = _run(w, x, to_gpu(bias), 1)
    rows = sample_indices(w.M, w.TP, 3, seed=1)
    cols = sample_indices(w.N, 1, 6, seed=2)
    D0 = _run(w, x, None, 1)
    expect = D0 + torch.from_numpy(bias).cuda()[None, None, :]
    assert torch.equal(D, expect)
    log("c3 with bias: max err", check_sampled(w, x, D, rows, cols, bias=bias))
