"""Seeded synthetic inputs for the TP-step GEMM, shared by the oracle's tests,
the GPU parity tests and the benchmark.

This module only *draws* operands; it holds none of the GEMM's arithmetic.
Quantisation of the drawn fp32 values to bf16 / OCP e4m3fn is done with
PyTorch's own CPU casts (round-to-nearest-even), so that the oracle (which
decodes the stored bytes with its own tables) and the HIP path consume the
exact same operand bytes.

Layouts (one GPU's share, batch index l outermost):
  A : L x M x K row-major (K contiguous)
  B : L x N x K row-major -- the K x N operand stored K-contiguous ("TN")
  C : L x M x N row-major
The five workloads are the per-GPU shares that the CUTLASS Distributed GEMM
example page, its pull-request page and the chunked all_gather+matmul blog
page describe (schedules AllGather1D_TilingCD_RotatingA/B and
ReduceScatter1D_TilingA/B_RotatingC, TP = number of steps).
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

SCHEDULES = ("AG_ROT_A", "AG_ROT_B", "RS_TILE_A_ROT_C", "RS_TILE_B_ROT_C", "MONOLITHIC")
# dtype name -> (input element, output/C element)
DTYPES = {
    "F32": ("f32", "f32"),
    "BF16_F32": ("bf16", "f32"),
    "BF16_BF16": ("bf16", "bf16"),
    "E4M3_BF16": ("e4m3", "bf16"),
    "E4M3_F32": ("e4m3", "f32"),
    "E4M3_E4M3": ("e4m3", "e4m3"),
}
E4M3_MAX = 448.0


@dataclass(frozen=True)
class Workload:
    name: str
    schedule: str
    dtype: str
    M: int
    N: int
    K: int
    L: int = 1
    TP: int = 8
    alpha: float = 1.0
    beta: float = 0.0
    # distribution of A/B/C entries: ("uniform", lo, hi) | ("normal", sigma)
    # | ("normal_amax448",)  (N(0,1) scaled so max|x| maps to 448, per-tensor)
    dist_ab: tuple = ("uniform", -1.0, 1.0)
    dist_c: tuple = ("uniform", -1.0, 1.0)
    seed_a: int = 1
    seed_b: int = 2
    seed_c: int = 3
    # seeds for independently drawn row blocks of A (config 2's two halves)
    seed_a_blocks: tuple = ()
    note: str = ""

    @property
    def in_dtype(self) -> str:
        return DTYPES[self.dtype][0]

    @property
    def out_dtype(self) -> str:
        return DTYPES[self.dtype][1]

    @property
    def flops(self) -> float:
        return 2.0 * self.M * self.N * self.K * self.L


# The five workloads.  Shapes are this GPU's totals over all TP steps.
CONFIGS = {
    # Tiny rotating-A all-gather+GEMM, TP=2, fp32, alpha=1.5 beta=0.5.
    "c1_tiny_ag_rot_a_f32": Workload(
        "c1_tiny_ag_rot_a_f32", "AG_ROT_A", "F32", 256, 256, 256, 1, 2, 1.5, 0.5,
        ("uniform", -1.0, 1.0), ("uniform", -1.0, 1.0), 101, 102, 103),
    # Chunked all_gather+matmul blog case on one GPU: gathered A 16384x8192
    # (two independent 8192x8192 U[0,1) halves), B 8192x8192 U[0,1), 8 chunks.
    "c2_blog_overlap_f32": Workload(
        "c2_blog_overlap_f32", "AG_ROT_A", "F32", 16384, 8192, 8192, 1, 8, 1.0, 0.0,
        ("uniform", 0.0, 1.0), ("uniform", 0.0, 1.0), 201, 203, 0, (201, 202)),
    # AllGather1D_TilingCD_RotatingA, one GPU's share at TP=8 of <16384,106496,16384>.
    "c3_ag_rot_a_bf16_tp8": Workload(
        "c3_ag_rot_a_bf16_tp8", "AG_ROT_A", "BF16_F32", 16384, 13312, 16384, 1, 8, 1.0, 0.0,
        ("normal", 1.0 / 128.0), ("normal", 1.0 / 128.0), 301, 302, 0),
    # ReduceScatter1D_TilingA_RotatingC, 70B-like MLP down-projection share at TP=8.
    "c4_rs_tile_a_rot_c_bf16_tp8": Workload(
        "c4_rs_tile_a_rot_c_bf16_tp8", "RS_TILE_A_ROT_C", "BF16_F32", 8192, 8192, 3584, 1, 8,
        1.0, 1.0, ("normal", 0.02), ("normal", 0.02), 401, 402, 403),
    # AllGather1D_TilingCD_RotatingB, 405B-like gate+up share at TP=8, e4m3 in, bf16 out.
    "c5_ag_rot_b_e4m3_tp8": Workload(
        "c5_ag_rot_b_e4m3_tp8", "AG_ROT_B", "E4M3_BF16", 8192, 13312, 16384, 1, 8, 1.0, 0.0,
        ("normal_amax448",), ("normal", 1.0), 501, 502, 0),
}
CONFIG_ORDER = list(CONFIGS)


@dataclass
class Inputs:
    """Operand bytes as numpy arrays.  bf16 is stored as uint16, e4m3fn as uint8."""
    A: np.ndarray
    B: np.ndarray
    C: Optional[np.ndarray]
    scale_a: float = 1.0
    scale_b: float = 1.0
    meta: dict = field(default_factory=dict)


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _draw_f32(dist: tuple, shape, seed: int) -> np.ndarray:
    g = _rng(seed)
    kind = dist[0]
    if kind == "uniform":
        lo, hi = np.float32(dist[1]), np.float32(dist[2])
        u = g.random(shape, dtype=np.float32)
        return (lo + (hi - lo) * u).astype(np.float32)
    if kind in ("normal", "normal_amax448"):
        sigma = np.float32(dist[1]) if kind == "normal" else np.float32(1.0)
        return (g.standard_normal(shape, dtype=np.float32) * sigma).astype(np.float32)
    raise ValueError(f"unknown distribution {dist!r}")


def _to_bf16_bits(x: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _to_e4m3_bits(x: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    t = t.clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def _encode(x: np.ndarray, elem: str, dist: tuple):
    """Returns (stored array, per-tensor dequant scale)."""
    if elem == "f32":
        return x.astype(np.float32), 1.0
    if dist[0] == "normal_amax448":
        amax = np.float32(np.max(np.abs(x)))
        s = np.float32(amax / np.float32(E4M3_MAX))
        x = (x / s).astype(np.float32)
        scale = float(s)
    else:
        scale = 1.0
    if elem == "bf16":
        return _to_bf16_bits(x), scale
    if elem == "e4m3":
        return _to_e4m3_bits(x), scale
    raise ValueError(elem)


def generate(w: Workload, need_c: Optional[bool] = None) -> Inputs:
    """Draw A (LxMxK), B (LxNxK) and C (LxMxN, only when beta != 0 or asked)."""
    L, M, N, K = w.L, w.M, w.N, w.K
    if w.seed_a_blocks:
        nb = len(w.seed_a_blocks)
        if M % nb:
            raise ValueError("M must split evenly into the independently drawn blocks")
        a32 = np.concatenate(
            [_draw_f32(w.dist_ab, (L, M // nb, K), s) for s in w.seed_a_blocks], axis=1)
    else:
        a32 = _draw_f32(w.dist_ab, (L, M, K), w.seed_a)
    A, sa = _encode(a32, w.in_dtype, w.dist_ab)
    del a32
    b32 = _draw_f32(w.dist_ab, (L, N, K), w.seed_b)
    B, sb = _encode(b32, w.in_dtype, w.dist_ab)
    del b32
    if need_c is None:
        need_c = w.beta != 0.0
    C = None
    if need_c:
        c32 = _draw_f32(w.dist_c, (L, M, N), w.seed_c)
        C, _ = _encode(c32, w.out_dtype, ("uniform", 0, 1))
    return Inputs(A, B, C, sa, sb, {"workload": w.name})


def small_case(name: str, schedule: str, dtype: str, M: int, N: int, K: int, L: int = 1,
               TP: int = 2, alpha: float = 1.0, beta: float = 0.0, seed: int = 7) -> Workload:
    """A parity-grid case with the distribution family its dtype's workload uses."""
    in_elem = DTYPES[dtype][0]
    if in_elem == "e4m3":
        dist_ab, dist_c = ("normal_amax448",), ("normal", 1.0)
    elif in_elem == "bf16":
        dist_ab, dist_c = ("normal", 1.0 / np.sqrt(max(K, 1))), ("normal", 0.02)
    else:
        dist_ab, dist_c = ("uniform", -1.0, 1.0), ("uniform", -1.0, 1.0)
    return Workload(name, schedule, dtype, M, N, K, L, TP, alpha, beta, dist_ab, dist_c,
                    seed * 10 + 1, seed * 10 + 2, seed * 10 + 3)


def with_schedule(w: Workload, schedule: str, TP: Optional[int] = None) -> Workload:
    return replace(w, schedule=schedule, TP=w.TP if TP is None else TP)
