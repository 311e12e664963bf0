"""MI355X (gfx950) TP-step GEMM: D = alpha*A*B + beta*C run as the
all-gather (rotating A or B) and reduce-scatter (rotating C) schedules of a
tensor-parallel layer, on one GPU's share of the work.

The compute path is the HIP library libdistgemm.so (C ABI in
include/distgemm.h); this package is its ctypes binding.  Importing it
fails if the library has not been built.
"""
from ._binding import (  # noqa: F401
    C_FUNCTIONS,
    DTYPES,
    ELEM_BYTES,
    LIB_PATH,
    OPTIONS,
    SCHEDULES,
    DistGemmError,
    Plan,
    dist_gemm_destroy,
    dist_gemm_device_errors,
    dist_gemm_fused_tables,
    dist_gemm_plan,
    dist_gemm_plan_steps,
    dist_gemm_run,
    dist_gemm_run_ag,
    dist_gemm_run_noalloc,
    dist_gemm_set_bias,
    dist_gemm_set_option,
    dist_gemm_set_result_scale,
    dist_gemm_set_scales,
    dist_gemm_step_table,
    dist_gemm_step_times,
    dist_gemm_step_timeline,
    lib,
)
