"""GPU tests of the half-height tail tiles (DIST_GEMM_OPT_HALF_TILES).

When the last round of an XCD's (single launch: a work queue's) tiles fills
at most half of its CUs, each of those tiles runs as two 128 x 256 halves.
Every element of D is produced by the same MFMA instructions in the same K
order either way, so a run with half tiles must equal the run without bit
for bit, for every element type, with and without C, with ragged edges;
the small cases are also compared with the oracle.

Shapes, with 256 x 256 tiles, 8 XCDs of 32 CUs and 8 queues of 32
workgroups:
* 600 x 520: 9 tiles, one or two per XCD: every tile is split.
* 4000 x 5000: 320 tiles, 40 per XCD or queue: the last 8 of each split.
* 16384 x 5376: 1344 tiles, 168 per queue: the last 8 of each split;
  8192 x 4864: 608 tiles, 76 per queue: the last 12.
* 8192 x 13312 (the e4m3 gate/up projection share): 1664 tiles, 208 per
  XCD or queue: the last 16 of each split.
"""
import pytest

import workloads
from gpu_helpers import check_full, log, run_plan, to_gpu

pytestmark = pytest.mark.gpu

DTYPES = ["F32", "BF16_F32", "BF16_BF16", "E4M3_BF16", "E4M3_F32", "E4M3_E4M3"]


def _both(w, x, schedule=None, TP=None, execution=1):
    dev = (to_gpu(x.A), to_gpu(x.B), to_gpu(x.C))
    on = run_plan(w, x, schedule=schedule, TP=TP, dev=dev, options={"EXECUTION": execution, "HALF_TILES": 1})
    off = run_plan(w, x, schedule=schedule, TP=TP, dev=dev, options={"EXECUTION": execution, "HALF_TILES": 0})
    return on, off


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("beta", [0.0, 0.5])
def test_every_tile_split_matches_whole_tiles_and_oracle(dtype, beta):
    import torch
    w = workloads.small_case(f"half_mono_{dtype}_{beta}", "MONOLITHIC", dtype, 600, 520, 272, 1, 1, 1.5, beta,
                             seed=31)
    x = workloads.generate(w)
    log("case", w.name)
    on, off = _both(w, x, schedule="MONOLITHIC", TP=1)
    assert torch.equal(on, off)
    check_full(w, x, on, schedule="MONOLITHIC", TP=1)


@pytest.mark.parametrize("execution", [1, 0])
@pytest.mark.parametrize("sched,dtype,beta", [
    ("AG_ROT_A", "BF16_BF16", 0.0),
    ("RS_TILE_B_ROT_C", "E4M3_F32", 1.0),
    ("AG_ROT_B", "E4M3_BF16", 0.0),
    ("RS_TILE_A_ROT_C", "BF16_F32", 1.0),
    ("AG_ROT_A", "F32", 0.5),
])
def test_small_schedules_with_split_tiles(execution, sched, dtype, beta):
    import torch
    w = workloads.small_case(f"half_{sched}_{dtype}", sched, dtype, 600, 520, 272, 1, 4, 1.0, beta, seed=37)
    x = workloads.generate(w)
    log("case", w.name, "execution", execution)
    on, off = _both(w, x, execution=execution)
    assert torch.equal(on, off)
    check_full(w, x, on)


@pytest.mark.parametrize("sched,dtype,M,N,K,beta", [
    ("MONOLITHIC", "BF16_BF16", 4000, 5000, 512, 0.0),
    ("MONOLITHIC", "BF16_F32", 4000, 5000, 512, 0.5),
    ("AG_ROT_A", "BF16_F32", 4000, 5000, 1024, 0.0),
    ("AG_ROT_A", "BF16_F32", 16384, 5376, 2048, 0.0),       # in-loop copies
    ("RS_TILE_A_ROT_C", "BF16_F32", 8192, 4864, 2048, 1.0),  # in-loop copies
    ("AG_ROT_B", "E4M3_BF16", 8192, 13312, 1024, 0.0),
    ("MONOLITHIC", "E4M3_BF16", 8192, 13312, 1024, 0.0),
])
def test_last_round_split_matches_whole_tiles(sched, dtype, M, N, K, beta):
    import torch
    TP = 1 if sched == "MONOLITHIC" else 8
    w = workloads.small_case(f"half_tail_{sched}_{dtype}_{M}x{N}x{K}", sched, dtype, M, N, K, 1, TP, 1.0, beta,
                             seed=41)
    x = workloads.generate(w)
    log("case", w.name)
    on, off = _both(w, x)
    assert torch.equal(on, off)


@pytest.mark.parametrize("sched,dtype,beta", [
    ("AG_ROT_A", "BF16_F32", 0.0),
    ("RS_TILE_B_ROT_C", "E4M3_BF16", 1.0),
])
def test_batched_split_tiles(sched, dtype, beta):
    # L = 3 batches of 600 x 520: the single launch's queues hold 27 tiles of
    # three batches, every one split; the monolithic GEMM splits only L = 1
    import torch
    w = workloads.small_case(f"half_batched_{sched}_{dtype}", sched, dtype, 600, 520, 272, 3, 4, 1.0, beta,
                             seed=43)
    x = workloads.generate(w)
    log("case", w.name)
    on, off = _both(w, x)
    assert torch.equal(on, off)
    check_full(w, x, on)


def test_half_tiles_option_values():
    import communication_tensor_gemm_amd as dg
    with dg.Plan(256, 256, 64, 1, 2, "AG_ROT_A", "BF16_F32") as p:
        p.set_option("HALF_TILES", 0)
        p.set_option("HALF_TILES", 1)
        for v in (-1, 2):
            with pytest.raises(dg.DistGemmError) as ei:
                p.set_option("HALF_TILES", v)
            assert ei.value.status == -1
