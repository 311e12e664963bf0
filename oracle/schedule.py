"""Step tables of the TP schedules, for one GPU of rank r in a group of S.

Schedules (names from the CUTLASS Distributed GEMM example page, section
"Trying out other schedules"; TP, the number of GPUs, is also the number of
steps, section of the same page on changing TP):

  AG_ROT_A        AllGather1D_TilingCD_RotatingA: A is split into S row
                  shards that rotate; B stays; step s writes the row block of
                  C/D that its A shard produces.
  AG_ROT_B        AllGather1D_TilingCD_RotatingB: B is split into S column
                  shards that rotate; A stays; step s writes a column block.
  RS_TILE_A_ROT_C ReduceScatter1D_TilingA_RotatingC: A is tiled into S row
                  chunks; the partial C chunk rotates and the epilogue adds
                  it with beta (the pull-request page: the epilogue source
                  serves as the communication buffer).
  RS_TILE_B_ROT_C ReduceScatter1D_TilingB_RotatingC: the same over column
                  chunks of B, C and D.
  MONOLITHIC      one step over the whole problem (the single-device GEMM
                  that the example's reference check compares against).

Rotation order.  The CUTLASS pages do not state it.  The PyTorch
symmetric-memory page fixes one: the all-gather consumer takes its own shard
first and then shard (step + rank) mod S (_pipelined_all_gather_and_consume);
the reduce-scatter producer makes chunk (rank + step) mod S at steps
1..S-1 and its own chunk last (_pipelined_produce_and_all2all).  This module
uses those orders.  Step 0 of every rotating schedule uses the GPU's local
operand in place; steps 1..S-1 consume an operand that had to be brought in
("staged").  The result does not depend on the order.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List

ROTATING = ("AG_ROT_A", "AG_ROT_B", "RS_TILE_A_ROT_C", "RS_TILE_B_ROT_C")


@dataclass(frozen=True)
class Step:
    s: int        # step index
    shard: int    # shard / chunk index consumed or produced
    m0: int
    m1: int
    n0: int
    n1: int
    staged: bool  # operand of this step arrives by a copy (not local)


def steps(schedule: str, M: int, N: int, S: int, rank: int = 0) -> List[Step]:
    if S < 1:
        raise ValueError("S must be >= 1")
    if schedule == "MONOLITHIC":
        return [Step(0, 0, 0, M, 0, N, False)]
    if schedule not in ROTATING:
        raise ValueError(f"unknown schedule {schedule}")
    by_rows = schedule in ("AG_ROT_A", "RS_TILE_A_ROT_C")
    extent = M if by_rows else N
    if extent % S:
        raise ValueError(f"{'M' if by_rows else 'N'}={extent} is not divisible by S={S}")
    w = extent // S
    out = []
    for s in range(S):
        if schedule.startswith("AG"):
            j = (rank + s) % S          # own shard first, then (step + rank) mod S
        else:
            j = (rank + s + 1) % S      # other chunks first, own chunk last
        lo, hi = j * w, (j + 1) * w
        if by_rows:
            out.append(Step(s, j, lo, hi, 0, N, s > 0))
        else:
            out.append(Step(s, j, 0, M, lo, hi, s > 0))
    return out


def local_problem(schedule: str, M: int, N: int, K: int, S: int):
    """Shape (m, n, k) of one step's GEMM."""
    st = steps(schedule, M, N, S)[0]
    return (st.m1 - st.m0, st.n1 - st.n0, K)
