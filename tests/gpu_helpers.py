"""Helpers for the GPU tests: upload seeded operand bytes, run a plan through
the C ABI, and compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np

import workloads
from oracle import codecs, gemm, parity

TORCH_STORE = {"f32": ("float32", np.float32), "bf16": ("int16", np.int16), "e4m3": ("uint8", np.uint8)}


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_gpu(arr):
    import torch
    if arr is None:
        return None
    if arr.dtype == np.uint16:
        arr = arr.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def empty_out(w: workloads.Workload, fill=np.nan):
    import torch
    shape = (w.L, w.M, w.N)
    if w.out_dtype == "f32":
        return torch.full(shape, float(fill), dtype=torch.float32, device="cuda")
    if w.out_dtype == "e4m3":
        # e4m3fn stored as uint8 bit patterns; 0x7F is NaN
        return torch.full(shape, 0x7F, dtype=torch.uint8, device="cuda")
    # bf16 stored as int16 bit patterns; 0x7FC0 is a NaN pattern
    return torch.full(shape, 0x7FC0, dtype=torch.int16, device="cuda")


def from_gpu_out(t, out_elem):
    a = t.cpu().numpy()
    if out_elem == "f32":
        return a.astype(np.float64)
    if out_elem == "e4m3":
        return codecs.e4m3_to_f64(a.view(np.uint8))
    return codecs.bf16_to_f64(a.view(np.uint16))


def run_plan(w: workloads.Workload, x: workloads.Inputs, schedule=None, TP=None, dev=None,
             out=None, options=None, alpha=None, beta=None, result_scale=None):
    """Run one dist_gemm_run and synchronize.  Returns the output tensor."""
    import torch
    import communication_tensor_gemm_amd as dg
    schedule = schedule or w.schedule
    TP = w.TP if TP is None else TP
    alpha = w.alpha if alpha is None else alpha
    beta = w.beta if beta is None else beta
    if dev is None:
        dev = (to_gpu(x.A), to_gpu(x.B), to_gpu(x.C))
    A, B, C = dev
    D = empty_out(w) if out is None else out
    with dg.Plan(w.M, w.N, w.K, w.L, TP, schedule, w.dtype) as plan:
        if w.in_dtype == "e4m3":
            plan.set_scales(x.scale_a, x.scale_b)
        if result_scale is not None:
            plan.set_result_scale(result_scale)
        for k, v in (options or {}).items():
            plan.set_option(k, v)
        plan.run(A, B, C if beta != 0.0 else None, D, alpha, beta)
        torch.cuda.synchronize()
    return D


def check_full(w, x, D, schedule=None, TP=None, alpha=None, beta=None, bias=None, result_scale=1.0):
    """Element-by-element comparison with the full oracle.  Returns max err.
    bias: the bias bytes (N output elements) the run used, or None."""
    schedule = schedule or w.schedule
    TP = w.TP if TP is None else TP
    alpha = w.alpha if alpha is None else alpha
    beta = w.beta if beta is None else beta
    Dstar = gemm.dist_gemm(x.A, x.B, x.C if beta != 0 else None, alpha, beta, schedule,
                           TP if schedule != "MONOLITHIC" else 1, w.in_dtype, w.out_dtype,
                           x.scale_a, x.scale_b, bias=bias, result_scale=result_scale)
    bdec = None if bias is None else codecs.decode(np.asarray(bias).reshape(-1), w.out_dtype)
    got = from_gpu_out(D, w.out_dtype)
    worst = 0.0
    for l in range(w.L):
        a = codecs.decode(x.A[l], w.in_dtype) * x.scale_a
        b = codecs.decode(x.B[l], w.in_dtype) * x.scale_b
        c = None if beta == 0 else codecs.decode(x.C[l], w.out_dtype)
        ok, mx, tight, _ = parity.check(got[l], Dstar[l], np.linalg.norm(a, axis=1),
                                        np.linalg.norm(b, axis=1), alpha, beta, c,
                                        w.in_dtype, w.out_dtype, bdec, result_scale)
        assert ok, f"{w.name} batch {l}: max normalised error {mx}"
        assert tight, f"{w.name} batch {l}: tight bar failed (max err {mx})"
        worst = max(worst, mx)
    return worst


def sample_indices(extent, steps, per_step, seed, tile=256):
    """Rows (or columns) covering every step block: its first and last index,
    indices either side of 256-tile edges inside it, and random ones."""
    g = np.random.default_rng(seed)
    w = extent // steps
    idx = set()
    for s in range(steps):
        lo, hi = s * w, (s + 1) * w
        idx.update({lo, hi - 1})
        for e in range(lo + tile, hi, tile * max(1, (hi - lo) // (tile * 4))):
            idx.update({e - 1, e})
        idx.update(g.integers(lo, hi, per_step).tolist())
    return np.array(sorted(i for i in idx if 0 <= i < extent), dtype=np.int64)


def check_sampled(w, x, D, rows, cols, schedule=None, TP=None, bias=None):
    schedule = schedule or w.schedule
    TP = w.TP if TP is None else TP
    Dstar, rn, cn = gemm.dist_gemm_sampled(x.A, x.B, x.C, w.alpha, w.beta, schedule, TP,
                                           w.in_dtype, w.out_dtype, rows, cols, x.scale_a,
                                           x.scale_b, bias=bias)
    bdec = None if bias is None else codecs.decode(np.asarray(bias).reshape(-1), w.out_dtype)[cols]
    import torch
    ri = torch.from_numpy(rows).cuda()
    ci = torch.from_numpy(cols).cuda()
    sub = D[0].index_select(0, ri).index_select(1, ci)
    got = from_gpu_out(sub, w.out_dtype)
    c = None
    if w.beta != 0:
        c = codecs.decode(x.C[0][np.ix_(rows, cols)], w.out_dtype)
    ok, mx, tight, _ = parity.check(got, Dstar, rn, cn, w.alpha, w.beta, c, w.in_dtype,
                                    w.out_dtype, bdec)
    assert ok, f"{w.name}: sampled max normalised error {mx}"
    assert tight, f"{w.name}: sampled tight bar failed (max err {mx})"
    return mx
