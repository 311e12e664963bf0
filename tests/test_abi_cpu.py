"""CPU checks of the C ABI: the library loads, exports every function that
include/distgemm.h declares, and its host-only step table agrees with the
oracle's (no GPU work is issued here)."""
import ctypes
import os
import re

import pytest

import communication_tensor_gemm_amd as dg
from oracle import schedule as oracle_schedule

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "distgemm.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dist_gemm_\w+)\s*\(", text)))


def test_header_declarations_are_exported():
    declared = _declared_functions()
    assert len(declared) >= 10
    lib = ctypes.CDLL(dg.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name
    assert sorted(dg.C_FUNCTIONS) == declared


def test_status_strings():
    assert dg.lib.dist_gemm_status_string(0) == b"DIST_GEMM_OK"
    assert dg.lib.dist_gemm_status_string(-2) == b"DIST_GEMM_ERR_SHAPE"


@pytest.mark.parametrize("sched", list(dg.SCHEDULES))
@pytest.mark.parametrize("S", [1, 2, 3, 8])
def test_step_table_matches_oracle(sched, S):
    M, N, K = 48 * S, 40 * S, 64
    got = dg.dist_gemm_step_table(M, N, K, 1, S, sched, "BF16_F32")
    ref = oracle_schedule.steps(sched, M, N, S)
    assert len(got) == len(ref)
    for g, r in zip(got, ref):
        step, shard, staged, slot, m0, m1, n0, n1 = g
        assert (step, shard, staged, m0, m1, n0, n1) == (r.s, r.shard, r.staged, r.m0, r.m1, r.n0, r.n1)
        assert slot == (shard if staged else -1)


def test_p2_local_shape_from_step_table():
    st = dg.dist_gemm_step_table(16384, 13312, 16384, 1, 8, "AG_ROT_A", "BF16_F32")
    assert all((s[5] - s[4], s[7] - s[6]) == (2048, 13312) for s in st)


@pytest.mark.parametrize("args,status", [
    ((0, 8, 16, 1, 1, "MONOLITHIC", "F32"), -1),          # M = 0
    ((8, 8, 16, 1, 0, "AG_ROT_A", "F32"), -1),            # TP = 0
    ((8, 8, 16, 1, 2, 9, "F32"), -1),                      # bad schedule
    ((8, 8, 16, 1, 2, "AG_ROT_A", 17), -1),               # bad dtype
    ((10, 8, 16, 1, 4, "AG_ROT_A", "F32"), -2),           # M % TP
    ((8, 10, 16, 1, 4, "RS_TILE_B_ROT_C", "F32"), -2),    # N % TP
    ((8, 8, 6, 1, 2, "AG_ROT_A", "BF16_F32"), -2),        # K * 2 bytes not a multiple of 16
    ((8, 8, 8, 1, 2, "AG_ROT_A", "E4M3_BF16"), -2),       # K * 1 byte not a multiple of 16
    ((8, 8, 1 << 23, 1, 2, "AG_ROT_A", "BF16_F32"), -2),  # 256 rows of K span >= 2 GiB
    ((8, 8, 16, 70000, 2, "AG_ROT_A", "F32"), -2),        # L too large
])
def test_validation_errors(args, status):
    with pytest.raises(dg.DistGemmError) as ei:
        dg.dist_gemm_step_table(*args)
    assert ei.value.status == status
    assert dg.lib.dist_gemm_last_error(None)


def test_null_handles_are_rejected_without_gpu():
    assert dg.lib.dist_gemm_set_scales(None, 1.0, 1.0) == -1
    assert dg.lib.dist_gemm_set_bias(None, None) == -1
    assert dg.lib.dist_gemm_set_option(None, 0, 1) == -1
    assert dg.lib.dist_gemm_run(None, None, None, None, None, 1.0, 0.0, None) == -1
    assert dg.lib.dist_gemm_run_ag(None, None, None, None, None, None, 1.0, 0.0, None) == -1
    assert dg.lib.dist_gemm_destroy(None) == 0
    n = ctypes.c_int(0)
    assert dg.lib.dist_gemm_step_table(8, 8, 16, 1, 2, 0, 0, None, None) == -1
    assert dg.lib.dist_gemm_plan_steps(None, None, ctypes.byref(n)) == -1
    assert dg.lib.dist_gemm_step_times(None, None, ctypes.byref(n)) == -1
    assert dg.lib.dist_gemm_step_timeline(None, None, ctypes.byref(n)) == -1
    c = ctypes.c_int64(0)
    assert dg.lib.dist_gemm_device_errors(None, ctypes.byref(c)) == -1
    assert dg.lib.dist_gemm_set_result_scale(None, 1.0) == -1
    for opt in range(13):
        assert dg.lib.dist_gemm_set_option(None, opt, 1) == -1


def test_single_hip_runtime_in_process():
    """The package must not bring a second libamdhip64 next to torch's."""
    import subprocess
    import sys
    code = ("import communication_tensor_gemm_amd, torch;"
            "m=open('/proc/self/maps').read();"
            "print(len({l.split()[-1] for l in m.splitlines() if 'libamdhip64' in l}))")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT)
    assert out.stdout.strip() == "1", out.stdout + out.stderr
