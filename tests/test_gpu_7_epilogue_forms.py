"""The epilogue's forms compute the same arithmetic and must agree bit for bit:
fp32 output staged through LDS with 16-byte stores, C streamed into LDS by
DMA, bf16 output staged with 8-byte stores, and the element-wise form that
buffers without that alignment take.  Each case runs once with D (and C)
aligned and once with both one element past an aligned address; the two
results must be identical and match the oracle.
"""
import numpy as np
import pytest

import workloads
from gpu_helpers import check_full, empty_out, log, run_plan, to_gpu

CASES = [
    ("AG_ROT_A", "BF16_F32", 1.0, 0.0),         # staged fp32, no C
    ("AG_ROT_A", "BF16_F32", 1.25, 0.5),        # C through LDS
    ("RS_TILE_A_ROT_C", "BF16_F32", 1.0, 1.0),  # staged partials as C
    ("AG_ROT_B", "BF16_BF16", 1.0, 0.0),        # staged bf16
    ("AG_ROT_B", "E4M3_BF16", 1.0, 0.0),        # staged bf16, e4m3 unit
    ("AG_ROT_A", "E4M3_F32", 1.0, 0.5),         # C through LDS, e4m3 unit
    ("AG_ROT_A", "F32", 1.0, 0.5),              # C through LDS, fp32 unit
]


def _offset_like(t):
    """A tensor of t's shape and dtype that starts one element into a fresh
    buffer (so its address is not 8- or 16-byte aligned), filled as t."""
    import torch
    flat = torch.empty(t.numel() + 8, dtype=t.dtype, device=t.device)
    v = flat[1:1 + t.numel()].view(t.shape)
    v.copy_(t)
    return v


def _bits(t):
    import torch
    return t.view(torch.int32) if t.dtype == torch.float32 else t


@pytest.mark.gpu
@pytest.mark.parametrize("execution", [0, 1])
@pytest.mark.parametrize("sched,dtype,alpha,beta", CASES)
def test_epilogue_forms_agree(sched, dtype, alpha, beta, execution):
    import torch
    # 512 x 1024 x 256 at TP=2: whole 256 x 256 tiles in every step
    w = workloads.small_case(f"epi_{sched}_{dtype}", sched, dtype, 512, 1024, 256, 1, 2,
                             alpha, beta, seed=71)
    x = workloads.generate(w)
    log(f"case {w.name} execution {execution} alpha {alpha} beta {beta}")
    A, B, C = to_gpu(x.A), to_gpu(x.B), to_gpu(x.C)
    opts = {"EXECUTION": execution}
    d_aligned = run_plan(w, x, dev=(A, B, C), out=empty_out(w), options=opts)
    c_off = None if C is None else _offset_like(C)
    d_off = _offset_like(empty_out(w))
    assert d_off.data_ptr() % 8 != 0
    run_plan(w, x, dev=(A, B, c_off), out=d_off, options=opts)
    torch.cuda.synchronize()
    same = torch.equal(_bits(d_aligned), _bits(d_off))
    if not same:
        diff = (_bits(d_aligned) != _bits(d_off)).nonzero()
        log(f"first differing elements: {diff[:5].tolist()}")
    assert same, f"{w.name}: aligned and element-wise epilogues differ"
    err = check_full(w, x, d_aligned)
    log(f"  max normalised error {err:.3e}")
