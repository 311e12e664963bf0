"""Pins for the oracle's step-scheduled GEMM (CPU only).

* brute force in exact rational arithmetic on tiny inputs, with operands
  decoded by PyTorch (not by the oracle's codecs), for every schedule and
  element type;
* the invariant that the step schedule equals the unchunked GEMM;
* closed forms of the epilogue: alpha=0 gives beta*C, B=I gives
  alpha*A + beta*C, linearity in (alpha, beta), TP=1 is the plain GEMM;
* the step table covers D exactly once, own shard first for the all-gather
  schedules and own chunk last for the reduce-scatter ones;
* the per-step shapes and TFLOPS that the Distributed GEMM pull-request page
  prints for TP=8 and TP=4;
* the output mean that the chunked all_gather+matmul blog page prints.
"""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import workloads
from oracle import gemm, schedule

SCHEDS = ["AG_ROT_A", "AG_ROT_B", "RS_TILE_A_ROT_C", "RS_TILE_B_ROT_C", "MONOLITHIC"]


def _inputs(dtype, M, N, K, L=1, beta=0.5, seed=3):
    w = workloads.small_case("t", "MONOLITHIC", dtype, M, N, K, L, 1, 1.25, beta, seed)
    return w, workloads.generate(w, need_c=True)


def _torch_decode(arr, elem):
    """Library decode, independent of oracle.codecs."""
    if elem == "f32":
        return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).double().numpy()
    if elem == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).double().numpy()
    if elem == "e4m3":
        return torch.from_numpy(np.ascontiguousarray(arr)).view(torch.float8_e4m3fn).double().numpy()
    raise ValueError(elem)


def _brute(A, B, C, alpha, beta, in_elem, out_elem, sa, sb):
    a = _torch_decode(A, in_elem)
    b = _torch_decode(B, in_elem)
    c = _torch_decode(C, out_elem)
    L, M, K = a.shape
    N = b.shape[1]
    ex = np.empty((L, M, N), dtype=object)
    mag = np.empty((L, M, N), dtype=np.float64)
    fa, fb, fs = Fraction(alpha), Fraction(beta), Fraction(sa) * Fraction(sb)
    for l, i, j in itertools.product(range(L), range(M), range(N)):
        dot = sum((Fraction(float(a[l, i, k])) * Fraction(float(b[l, j, k])) for k in range(K)),
                  Fraction(0))
        ex[l, i, j] = fa * fs * dot + fb * Fraction(float(c[l, i, j]))
        mag[l, i, j] = abs(alpha) * sa * sb * float(np.abs(a[l, i]) @ np.abs(b[l, j])) \
            + abs(beta) * abs(float(c[l, i, j]))
    return ex, mag


TINY = [(1, 1, 1), (2, 3, 1), (4, 8, 3), (8, 4, 16), (16, 8, 32)]


@pytest.mark.parametrize("dtype", ["F32", "BF16_F32", "BF16_BF16", "E4M3_BF16"])
@pytest.mark.parametrize("sched", SCHEDS)
def test_brute_force_exact(dtype, sched):
    in_elem, out_elem = workloads.DTYPES[dtype]
    for (M, N, K) in TINY:
        for S in (1, 2, 4):
            ext = M if sched in ("AG_ROT_A", "RS_TILE_A_ROT_C") else N
            if sched != "MONOLITHIC" and ext % S:
                continue
            w, x = _inputs(dtype, M, N, K, L=2 if (M, N, K) == (4, 8, 3) else 1)
            D = gemm.dist_gemm(x.A, x.B, x.C, w.alpha, w.beta, sched, S, in_elem, out_elem,
                               x.scale_a, x.scale_b)
            ex, mag = _brute(x.A, x.B, x.C, w.alpha, w.beta, in_elem, out_elem, x.scale_a,
                             x.scale_b)
            bound = (K + 4) * 2.0 ** -53 * mag * 1.01
            for idx in np.ndindex(D.shape):
                err = abs(Fraction(float(D[idx])) - ex[idx])
                assert err <= Fraction(float(bound[idx])), (sched, dtype, M, N, K, S, idx)


@pytest.mark.parametrize("sched", SCHEDS[:4])
def test_schedule_equals_unchunked(sched):
    for dtype in ("F32", "BF16_F32", "E4M3_BF16"):
        in_elem, out_elem = workloads.DTYPES[dtype]
        w, x = _inputs(dtype, 48, 40, 37, L=2)
        ref = gemm.gemm_unchunked(x.A, x.B, x.C, w.alpha, w.beta, in_elem, out_elem,
                                  x.scale_a, x.scale_b)
        for S in (1, 2, 4, 8):
            D = gemm.dist_gemm(x.A, x.B, x.C, w.alpha, w.beta, sched, S, in_elem, out_elem,
                               x.scale_a, x.scale_b)
            a = _torch_decode(x.A, in_elem) * x.scale_a
            b = _torch_decode(x.B, in_elem) * x.scale_b
            mag = abs(w.alpha) * np.matmul(np.abs(a), np.abs(b).transpose(0, 2, 1)) \
                + abs(w.beta) * np.abs(_torch_decode(x.C, out_elem))
            assert np.all(np.abs(D - ref) <= 2 * 40 * 2.0 ** -53 * mag)


def test_alpha_zero_gives_beta_c_exactly():
    for dtype in ("F32", "BF16_F32", "E4M3_BF16"):
        in_elem, out_elem = workloads.DTYPES[dtype]
        w, x = _inputs(dtype, 32, 24, 40)
        for sched in SCHEDS:
            D = gemm.dist_gemm(x.A, x.B, x.C, 0.0, 0.75, sched, 4 if sched != "MONOLITHIC" else 1,
                               in_elem, out_elem, x.scale_a, x.scale_b)
            assert np.array_equal(D, 0.75 * _torch_decode(x.C, out_elem))


def test_identity_b_gives_alpha_a_plus_beta_c():
    # B = I (N == K): one nonzero product per element, so the result is exact
    g = np.random.default_rng(1)
    M = K = N = 16
    A = g.uniform(-1, 1, (1, M, K)).astype(np.float32)
    B = np.eye(N, K, dtype=np.float32)[None]
    C = g.uniform(-1, 1, (1, M, N)).astype(np.float32)
    for sched in SCHEDS:
        D = gemm.dist_gemm(A, B, C, 1.5, -0.25, sched, 4 if sched != "MONOLITHIC" else 1, "f32", "f32")
        expect = 1.5 * A.astype(np.float64) + (-0.25) * C.astype(np.float64)
        assert np.array_equal(D, expect)
    # e4m3 identity: code 0x38 is 1.0
    A8 = g.integers(0, 0x7E, (1, M, K)).astype(np.uint8)
    B8 = np.where(np.eye(N, K, dtype=bool), 0x38, 0x00).astype(np.uint8)[None]
    D = gemm.dist_gemm(A8, B8, None, 2.0, 0.0, "AG_ROT_B", 4, "e4m3", "bf16")
    assert np.array_equal(D, 2.0 * _torch_decode(A8, "e4m3"))


def test_linearity_in_alpha_beta():
    w, x = _inputs("F32", 24, 32, 20)
    D10 = gemm.dist_gemm(x.A, x.B, x.C, 1.0, 0.0, "RS_TILE_B_ROT_C", 4, "f32", "f32")
    D = gemm.dist_gemm(x.A, x.B, x.C, -2.5, 3.0, "RS_TILE_B_ROT_C", 4, "f32", "f32")
    expect = -2.5 * D10 + 3.0 * x.C.astype(np.float64)
    assert np.allclose(D, expect, rtol=1e-14, atol=1e-13)


def test_tp1_rotating_equals_monolithic_exactly():
    w, x = _inputs("BF16_F32", 40, 24, 64)
    mono = gemm.dist_gemm(x.A, x.B, x.C, 1.25, 0.5, "MONOLITHIC", 1, "bf16", "f32")
    for sched in SCHEDS[:4]:
        assert np.array_equal(gemm.dist_gemm(x.A, x.B, x.C, 1.25, 0.5, sched, 1, "bf16", "f32"), mono)


def test_beta_zero_does_not_read_c():
    w, x = _inputs("F32", 8, 8, 8)
    C = np.full_like(x.C, np.nan)
    D = gemm.dist_gemm(x.A, x.B, C, 1.0, 0.0, "AG_ROT_A", 2, "f32", "f32")
    assert np.all(np.isfinite(D))


@pytest.mark.parametrize("sched", SCHEDS)
@pytest.mark.parametrize("S", [1, 2, 3, 8])
def test_step_table_partitions_output(sched, S):
    M, N = 24 * S, 16 * S
    st = schedule.steps(sched, M, N, S)
    cover = np.zeros((M, N), dtype=np.int32)
    for s in st:
        cover[s.m0:s.m1, s.n0:s.n1] += 1
    assert np.all(cover == 1)
    if sched == "MONOLITHIC":
        assert len(st) == 1
        return
    assert [s.s for s in st] == list(range(S))
    assert sorted(s.shard for s in st) == list(range(S))
    assert [s.staged for s in st] == [False] + [True] * (S - 1)
    for rank in range(S):
        st_r = schedule.steps(sched, M, N, S, rank)
        if sched.startswith("AG"):
            assert st_r[0].shard == rank           # local shard consumed first
        else:
            assert st_r[-1].shard == rank          # own chunk produced last


def test_step_table_rejects_indivisible():
    with pytest.raises(ValueError):
        schedule.steps("AG_ROT_A", 10, 8, 4)
    with pytest.raises(ValueError):
        schedule.steps("RS_TILE_B_ROT_C", 8, 10, 4)


# Distributed GEMM pull-request page, the two printed runs: problem
# 16384 x 106496 x 16384 x 1; TP=8 -> local 2048 x 13312 x 16384, 9.16037 ms,
# 780.19 TFLOPS; TP=4 -> local 4096 x 26624 x 16384, 16.8623 ms, 847.67 TFLOPS.
@pytest.mark.parametrize("TP,local,ms,tflops", [
    (8, (2048, 13312, 16384), 9.16037, 780.19),
    (4, (4096, 26624, 16384), 16.8623, 847.67),
])
def test_printed_local_shapes_and_rates(TP, local, ms, tflops):
    M, Nglob, K = 16384, 106496, 16384
    Nloc = Nglob // TP           # B's column shard that stays on this GPU
    assert schedule.local_problem("AG_ROT_A", M, Nloc, K, TP) == local
    per, total = gemm.step_flops("AG_ROT_A", M, Nloc, K, TP)
    assert len(per) == TP
    assert round(total / (ms * 1e-3) / 1e12, 2) == tflops


def test_blog_output_mean():
    """Chunked all_gather+matmul blog page: U[0,1) inputs, K = 8192, printed
    output mean 2047.625...; the expectation is K * E[a] * E[b] = 2048."""
    w = workloads.CONFIGS["c2_blog_overlap_f32"]
    g = np.random.default_rng(11)
    # a 256 x 256 sample of the workload's output, drawn from both A halves
    K = w.K
    x = workloads.generate(workloads.Workload(
        "s", "AG_ROT_A", "F32", 512, 512, K, 1, 8, 1.0, 0.0, w.dist_ab, w.dist_c, 0, 203, 0,
        (201, 202)))
    rows = np.sort(g.choice(512, 256, replace=False))
    cols = np.sort(g.choice(512, 256, replace=False))
    D, rn, cn = gemm.dist_gemm_sampled(x.A, x.B, None, 1.0, 0.0, "AG_ROT_A", 8, "f32", "f32",
                                       rows, cols)
    assert abs(D.mean() - 2048.0) < 6.0
    assert abs(D.mean() - 2047.62548828125) < 6.0


def test_sampled_matches_full():
    w, x = _inputs("BF16_F32", 64, 48, 40, L=2)
    for sched in SCHEDS[:4]:
        full = gemm.dist_gemm(x.A, x.B, x.C, w.alpha, w.beta, sched, 4, "bf16", "f32")
        rows = [0, 5, 17, 63, 31]
        cols = [47, 0, 12, 13]
        D, rn, cn = gemm.dist_gemm_sampled(x.A, x.B, x.C, w.alpha, w.beta, sched, 4, "bf16", "f32",
                                           rows, cols, batch=1)
        assert np.allclose(D, full[1][np.ix_(rows, cols)], rtol=1e-13, atol=1e-15)
        assert np.allclose(rn, np.linalg.norm(_torch_decode(x.A, "bf16")[1][rows], axis=1))


def _bias_bytes(N, out_elem, seed):
    """A bias vector in the output element's storage (float32, or bf16 bits)."""
    v = np.random.default_rng(seed).standard_normal(N).astype(np.float32)
    if out_elem == "f32":
        return v
    return torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("dtype", ["F32", "BF16_F32", "BF16_BF16", "E4M3_BF16"])
@pytest.mark.parametrize("sched", SCHEDS)
def test_brute_force_exact_with_bias(dtype, sched):
    """The scaled-matmul bias: one value per output column, added to every row
    and batch; exact rational arithmetic, bias decoded by PyTorch."""
    in_elem, out_elem = workloads.DTYPES[dtype]
    for (M, N, K) in [(2, 3, 1), (4, 8, 3), (8, 4, 16)]:
        for S in (1, 2, 4):
            ext = M if sched in ("AG_ROT_A", "RS_TILE_A_ROT_C") else N
            if sched != "MONOLITHIC" and ext % S:
                continue
            w, x = _inputs(dtype, M, N, K, L=2)
            bias = _bias_bytes(N, out_elem, seed=M * 100 + N)
            D = gemm.dist_gemm(x.A, x.B, x.C, w.alpha, w.beta, sched, S, in_elem, out_elem,
                               x.scale_a, x.scale_b, bias=bias)
            ex, mag = _brute(x.A, x.B, x.C, w.alpha, w.beta, in_elem, out_elem, x.scale_a,
                             x.scale_b)
            bt = _torch_decode(bias, out_elem)
            bound = (K + 5) * 2.0 ** -53 * (mag + np.abs(bt)[None, None, :]) * 1.01
            for idx in np.ndindex(D.shape):
                exact = ex[idx] + Fraction(float(bt[idx[2]]))
                err = abs(Fraction(float(D[idx])) - exact)
                assert err <= Fraction(float(bound[idx])), (sched, dtype, M, N, K, S, idx)


def test_bias_alone_and_linearity():
    """alpha = beta = 0 leaves exactly the bias in every row; adding a bias
    shifts every column of D by exactly that value (bias and D in fp64)."""
    w, x = _inputs("BF16_BF16", 24, 40, 16, L=2)
    bias = _bias_bytes(40, "bf16", seed=9)
    bt = _torch_decode(bias, "bf16")
    for sched in SCHEDS:
        S = 4 if sched != "MONOLITHIC" else 1
        D0 = gemm.dist_gemm(x.A, x.B, x.C, 0.0, 0.0, sched, S, "bf16", "bf16", bias=bias)
        assert np.array_equal(D0, np.broadcast_to(bt, D0.shape))
        Dn = gemm.dist_gemm(x.A, x.B, x.C, 1.5, 0.5, sched, S, "bf16", "bf16")
        Db = gemm.dist_gemm(x.A, x.B, x.C, 1.5, 0.5, sched, S, "bf16", "bf16", bias=bias)
        assert np.allclose(Db - Dn, np.broadcast_to(bt, Dn.shape), rtol=0, atol=1e-12)
        un = gemm.gemm_unchunked(x.A, x.B, x.C, 1.5, 0.5, "bf16", "bf16", bias=bias)
        assert np.allclose(Db, un, rtol=1e-13, atol=1e-13)


def test_sampled_matches_full_with_bias():
    w, x = _inputs("BF16_F32", 64, 48, 40, L=2)
    bias = _bias_bytes(48, "f32", seed=4)
    for sched in SCHEDS[:4]:
        full = gemm.dist_gemm(x.A, x.B, x.C, w.alpha, w.beta, sched, 4, "bf16", "f32", bias=bias)
        rows = [0, 5, 17, 63, 31]
        cols = [47, 0, 12, 13]
        D, rn, cn = gemm.dist_gemm_sampled(x.A, x.B, x.C, w.alpha, w.beta, sched, 4, "bf16", "f32",
                                           rows, cols, batch=1, bias=bias)
        assert np.allclose(D, full[1][np.ix_(rows, cols)], rtol=1e-13, atol=1e-15)



@pytest.mark.parametrize("sched", ["RS_TILE_A_ROT_C", "RS_TILE_B_ROT_C"])
@pytest.mark.parametrize("op", ["avg", "sum"])
def test_reduce_scatter_chain_with_bias(sched, op):
    """The fused (scaled) matmul + reduce-scatter of the PyTorch
    symmetric-memory page reduces the ranks' scaled-matmul outputs, each of
    which includes the bias, with reduce_op sum or avg: the result is
    sum_r (A_r B_r + bias) or its mean.  Read here as a chain of this GPU's
    share over the TP ranks (beta = 1, each output the next rank's incoming
    partial, starting from zero), where avg passes alpha = 1/TP and the bias
    divided by TP.  The oracle chained that way must give the reduction
    written out from its definition, up to the fp32 storage of the partials."""
    TP, M, N, K = 4, 8, 12, 16
    g = np.random.default_rng(21)
    As = [g.standard_normal((1, M, K)).astype(np.float32) for _ in range(TP)]
    Bs = [g.standard_normal((1, N, K)).astype(np.float32) for _ in range(TP)]
    bias = g.standard_normal(N).astype(np.float32)
    div = TP if op == "avg" else 1
    part = np.zeros((1, M, N), dtype=np.float32)
    for r in range(TP):
        b = (bias.astype(np.float64) / div).astype(np.float32)
        part = gemm.round_output(gemm.dist_gemm(As[r], Bs[r], part, 1.0 / div, 1.0, sched, TP,
                                                "f32", "f32", rank=r, bias=b), "f32")
    want = np.zeros((M, N))
    for r in range(TP):
        want += As[r][0].astype(np.float64) @ Bs[r][0].astype(np.float64).T + bias.astype(np.float64)
    want /= div
    mag = sum(np.abs(As[r][0]).astype(np.float64) @ np.abs(Bs[r][0]).astype(np.float64).T
              + np.abs(bias) for r in range(TP)) / div
    assert np.all(np.abs(part[0] - want) <= 4 * TP * 2.0 ** -24 * mag)
    # and not the other reduction: avg and sum differ by a factor TP
    other = want * TP if op == "avg" else want / TP
    assert not np.allclose(part[0], other)


def _torch_e4m3_nearest(x):
    """Nearest e4m3fn value to each float64 x (ties to the even code), from
    torch's decoding of all 256 codes, clipped to +-448 (the saturating
    cast): a rounding written independently of the oracle's encoder."""
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    vals = codes.view(torch.float8_e4m3fn).double().numpy()
    fin = np.isfinite(vals)
    v, c = vals[fin], np.arange(256)[fin]
    out = np.empty_like(np.asarray(x, dtype=np.float64))
    for i, xi in enumerate(np.clip(np.asarray(x, dtype=np.float64).ravel(), -448.0, 448.0)):
        d = np.abs(v - xi)
        best = np.nonzero(d == d.min())[0]
        if len(best) > 1:   # a tie: the even code (mantissa bit 0 clear)
            best = [b for b in best if c[b] % 2 == 0]
        out.flat[i] = v[best[0]]
    return out


@pytest.mark.parametrize("sched", SCHEDS)
def test_brute_force_result_scale_e4m3_output(sched):
    """The scaled matmul with an fp8 output: D = round_e4m3(s * (alpha*sa*sb*A B
    + beta*C)), s the result scale; exact rational arithmetic for the sum,
    rounding checked against torch's decoded e4m3 values."""
    S = 2 if sched != "MONOLITHIC" else 1
    for M, N, K, s in ((4, 6, 32, 0.3), (8, 4, 16, -2.75), (2, 8, 64, 7.0)):
        w, x = _inputs("E4M3_E4M3", M, N, K, beta=0.5, seed=M * 10 + N)
        ex, mag = _brute(x.A, x.B, x.C, 1.25, 0.5, "e4m3", "e4m3", x.scale_a, x.scale_b)
        D = gemm.dist_gemm(x.A, x.B, x.C, 1.25, 0.5, sched, S, "e4m3", "e4m3", x.scale_a, x.scale_b,
                           result_scale=s)
        want = np.vectorize(float)(ex) * s
        assert np.all(np.abs(D - want) <= 4 * K * 2.0 ** -53 * abs(s) * mag + 1e-300)
        got = gemm.round_output(D, "e4m3")
        assert np.array_equal(got, _torch_e4m3_nearest(D))
        assert np.all(np.abs(got) <= 448.0)


def test_result_scale_saturates_the_fp8_cast():
    w, x = _inputs("E4M3_E4M3", 8, 8, 32, beta=0.0, seed=5)
    D1 = gemm.dist_gemm(x.A, x.B, None, 1.0, 0.0, "AG_ROT_A", 2, "e4m3", "e4m3", x.scale_a, x.scale_b)
    big = 2000.0 / np.abs(D1).max()
    D = gemm.dist_gemm(x.A, x.B, None, 1.0, 0.0, "AG_ROT_A", 2, "e4m3", "e4m3", x.scale_a, x.scale_b,
                       result_scale=big)
    r = gemm.round_output(D, "e4m3")
    assert np.abs(D).max() > 448.0
    assert np.all(r[np.abs(D) >= 448.0] == np.sign(D[np.abs(D) >= 448.0]) * 448.0)
