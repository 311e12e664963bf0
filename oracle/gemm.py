"""The step-scheduled fp64 GEMM  D = s * (alpha * (sa*A) * (sb*B) + beta * C (+ bias)).

Definition followed: the CUTLASS Distributed GEMM pages compare the
distributed result against a single-device GEMM with the epilogue scalars
alpha (default 1) and beta (default 0) (example page, "Getting started"); the
PyTorch symmetric-memory page defines the fused all-gather matmul as
all_gather then matmul, the fused matmul reduce-scatter as matmul then
reduce_scatter, and the scaled variants as _scaled_mm with per-tensor
scale_a / scale_b, an optional bias added to every row of the product, and
a result scale s for an fp8 output (the op schemas and their fallbacks; the
pages pass scale_result through to _scaled_mm without defining it, read
here as a factor on the whole result before its one rounding to the output
element, s = 1 for the other outputs).

The oracle walks the same step table as the GPU path: one numpy float64
matmul per step on that step's row or column block, the epilogue in fp64,
written into that block.  Rounding to the output element happens once, at the
end, in ``round_output``.

Operand layout: A is L x M x K, B is stored L x N x K (the logical K x N
operand with K contiguous), C and D are L x M x N; the optional bias is one
vector of N values in the output element type, the same for every row and
batch.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from . import codecs
from .schedule import steps as step_table


def decode_operands(A, B, C, in_elem: str, out_elem: str, scale_a: float = 1.0,
                    scale_b: float = 1.0):
    """Stored bytes -> fp64 values (Ahat, Bhat, Chat).  Scales applied in fp64."""
    Ah = codecs.decode(A, in_elem) * np.float64(scale_a)
    Bh = codecs.decode(B, in_elem) * np.float64(scale_b)
    Ch = None if C is None else codecs.decode(C, out_elem)
    return Ah, Bh, Ch


def _as3(x):
    return None if x is None else (x if x.ndim == 3 else x[None])


def _bias(bias, out_elem: str):
    return None if bias is None else codecs.decode(np.asarray(bias).reshape(-1), out_elem)


def dist_gemm(A, B, C, alpha: float, beta: float, schedule: str, S: int, in_elem: str,
              out_elem: str, scale_a: float = 1.0, scale_b: float = 1.0,
              rank: int = 0, bias=None, result_scale: float = 1.0) -> np.ndarray:
    """Unrounded fp64 D* of the whole schedule, shape L x M x N."""
    Ah, Bh, Ch = decode_operands(_as3(A), _as3(B), _as3(C), in_elem, out_elem, scale_a, scale_b)
    bh = _bias(bias, out_elem)
    L, M, K = Ah.shape
    N = Bh.shape[1]
    if beta != 0.0 and Ch is None:
        raise ValueError("beta != 0 needs C")
    D = np.empty((L, M, N), dtype=np.float64)
    for st in step_table(schedule, M, N, S, rank):
        for l in range(L):
            a = Ah[l, st.m0:st.m1, :]
            b = Bh[l, st.n0:st.n1, :]
            acc = a @ b.T                                   # fp64 dgemm of this step
            blk = np.float64(alpha) * acc
            if beta != 0.0:                                 # C is not read when beta == 0
                blk = blk + np.float64(beta) * Ch[l, st.m0:st.m1, st.n0:st.n1]
            if bh is not None:                              # bias: one value per column
                blk = blk + bh[st.n0:st.n1][None, :]
            D[l, st.m0:st.m1, st.n0:st.n1] = np.float64(result_scale) * blk
    return D


def dist_gemm_sampled(A, B, C, alpha: float, beta: float, schedule: str, S: int, in_elem: str,
                      out_elem: str, rows: Sequence[int], cols: Sequence[int],
                      scale_a: float = 1.0, scale_b: float = 1.0, batch: int = 0,
                      rank: int = 0, bias=None, result_scale: float = 1.0):
    """D* on the sub-grid rows x cols of batch `batch`, visiting the same steps.

    Only the sampled rows of A and columns of B are decoded, so this runs at
    full workload sizes.  Returns (D*, row_norms, col_norms) where the norms
    are the l2 norms of the decoded rows of A and columns of B (the
    normaliser of the parity metric)."""
    A3, B3, C3 = _as3(A), _as3(B), _as3(C)
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    M, N = A3.shape[1], B3.shape[1]
    a = codecs.decode(A3[batch][rows], in_elem) * np.float64(scale_a)
    b = codecs.decode(B3[batch][cols], in_elem) * np.float64(scale_b)
    c = None
    if beta != 0.0:
        c = codecs.decode(C3[batch][np.ix_(rows, cols)], out_elem)
    bh = None if bias is None else _bias(bias, out_elem)[cols]
    D = np.full((len(rows), len(cols)), np.nan, dtype=np.float64)
    for st in step_table(schedule, M, N, S, rank):
        ri = np.nonzero((rows >= st.m0) & (rows < st.m1))[0]
        ci = np.nonzero((cols >= st.n0) & (cols < st.n1))[0]
        if len(ri) == 0 or len(ci) == 0:
            continue
        acc = a[ri] @ b[ci].T
        blk = np.float64(alpha) * acc
        if beta != 0.0:
            blk = blk + np.float64(beta) * c[np.ix_(ri, ci)]
        if bh is not None:
            blk = blk + bh[ci][None, :]
        D[np.ix_(ri, ci)] = np.float64(result_scale) * blk
    return D, np.linalg.norm(a, axis=1), np.linalg.norm(b, axis=1)


def round_output(D: np.ndarray, out_elem: str) -> np.ndarray:
    return codecs.round_to(D, out_elem)


def gemm_unchunked(A, B, C, alpha: float, beta: float, in_elem: str, out_elem: str,
                   scale_a: float = 1.0, scale_b: float = 1.0, bias=None,
                   result_scale: float = 1.0) -> np.ndarray:
    """The same definition evaluated as one fp64 matmul per batch, no steps."""
    Ah, Bh, Ch = decode_operands(_as3(A), _as3(B), _as3(C), in_elem, out_elem, scale_a, scale_b)
    D = np.float64(alpha) * np.matmul(Ah, np.transpose(Bh, (0, 2, 1)))
    if beta != 0.0:
        D = D + np.float64(beta) * Ch
    if bias is not None:
        D = D + _bias(bias, out_elem)[None, None, :]
    return np.float64(result_scale) * D


def step_flops(schedule: str, M: int, N: int, K: int, S: int, L: int = 1):
    """Per-step and total algorithmic flops (2*m*n*k per multiply-add)."""
    per = [2.0 * (st.m1 - st.m0) * (st.n1 - st.n0) * K * L for st in step_table(schedule, M, N, S)]
    return per, float(sum(per))
