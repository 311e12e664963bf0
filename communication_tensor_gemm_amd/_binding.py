"""ctypes binding of libdistgemm.so: argument marshalling only.

Every name mirrors a C entry point of include/distgemm.h.  Device buffers may
be passed as integers (device addresses) or as torch tensors, whose
data_ptr() is passed; torch is used for nothing else.  There is no fallback:
if the shared library is missing, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdistgemm.so")

SCHEDULES = {"AG_ROT_A": 0, "AG_ROT_B": 1, "RS_TILE_A_ROT_C": 2, "RS_TILE_B_ROT_C": 3,
             "MONOLITHIC": 4}
DTYPES = {"F32": 0, "BF16_F32": 1, "BF16_BF16": 2, "E4M3_BF16": 3, "E4M3_F32": 4, "E4M3_E4M3": 5}
OPTIONS = {"COMPUTE_STREAMS": 0, "COPY_ENGINE": 1, "STEP_TIMING": 2, "COPY_STREAMS": 3,
           "STEP_GROUP": 4, "EXECUTION": 5, "QUEUES": 6, "COPY_CHUNK": 7, "WAIT_LIMIT_US": 8,
           "COPY_AHEAD": 9, "SHARED_A": 10, "COPY_DELAY_US": 11, "FAST_ACCUM": 12,
           "HALF_TILES": 13}
# bytes per element of (A/B, C/D) for each dtype
ELEM_BYTES = {"F32": (4, 4), "BF16_F32": (2, 4), "BF16_BF16": (2, 2), "E4M3_BF16": (1, 2),
              "E4M3_F32": (1, 4), "E4M3_E4M3": (1, 1)}
STATUS = {0: "OK", -1: "INVALID_ARG", -2: "SHAPE", -3: "UNSUPPORTED", -4: "OOM", -5: "HIP"}

# C functions declared in include/distgemm.h (checked by the CPU tests)
C_FUNCTIONS = ("dist_gemm_step_table", "dist_gemm_fused_tables", "dist_gemm_plan", "dist_gemm_set_scales", "dist_gemm_set_result_scale",
               "dist_gemm_set_bias",
               "dist_gemm_set_option", "dist_gemm_run", "dist_gemm_run_ag", "dist_gemm_run_noalloc",
               "dist_gemm_plan_steps", "dist_gemm_step_times", "dist_gemm_step_timeline", "dist_gemm_device_errors",
               "dist_gemm_destroy", "dist_gemm_last_error", "dist_gemm_status_string")


class DistGemmError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class Step(ctypes.Structure):
    _fields_ = [("step", ctypes.c_int32), ("shard", ctypes.c_int32), ("staged", ctypes.c_int32),
                ("slot", ctypes.c_int32), ("m0", ctypes.c_int64), ("m1", ctypes.c_int64),
                ("n0", ctypes.c_int64), ("n1", ctypes.c_int64)]

    def as_tuple(self):
        return (self.step, self.shard, bool(self.staged), self.slot, self.m0, self.m1, self.n0,
                self.n1)


class FusedInfo(ctypes.Structure):
    _fields_ = [("n_strips", ctypes.c_int32), ("n_segs", ctypes.c_int32), ("LG", ctypes.c_int32),
                ("cols", ctypes.c_int32), ("strided", ctypes.c_int32), ("loop", ctypes.c_int32),
                ("n_list0", ctypes.c_int32), ("n_list1", ctypes.c_int32), ("n_local", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("strip_bytes", ctypes.c_int64), ("ext", ctypes.c_int64),
                ("row_bytes", ctypes.c_int64), ("height", ctypes.c_int64), ("loop_capacity", ctypes.c_int64)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python communication_tensor_gemm_amd/build.py`")
    # One HIP runtime per process: torch's ROCm build loads its own
    # libamdhip64 (soname libamdhip64.so.7) through an unversioned dependency.
    # Loading torch first makes this library's libamdhip64.so.7 dependency
    # resolve to that same runtime; loading it first would bring in a second
    # runtime alongside torch's, and one of the two then sees no device.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    lib.dist_gemm_step_table.argtypes = [i64, i64, i64, i64, i32, i32, i32,
                                         ctypes.POINTER(Step), ctypes.POINTER(i32)]
    lib.dist_gemm_fused_tables.argtypes = [i64, i64, i64, i64, i32, i32, i32, i32, i32, i32, i32, i64, i32,
                                           ctypes.POINTER(FusedInfo), vp, vp, vp, vp]
    lib.dist_gemm_plan.argtypes = [i64, i64, i64, i64, i32, i32, i32, ctypes.POINTER(vp)]
    lib.dist_gemm_set_scales.argtypes = [vp, ctypes.c_float, ctypes.c_float]
    lib.dist_gemm_set_bias.argtypes = [vp, vp]
    lib.dist_gemm_set_result_scale.argtypes = [vp, ctypes.c_float]
    lib.dist_gemm_set_option.argtypes = [vp, i32, i64]
    lib.dist_gemm_run.argtypes = [vp, vp, vp, vp, vp, ctypes.c_float, ctypes.c_float, vp]
    lib.dist_gemm_run_ag.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_float, ctypes.c_float, vp]
    f32 = ctypes.c_float
    lib.dist_gemm_run_noalloc.argtypes = [i64, i64, i64, i64, i32, i32, i32, vp, vp, vp, vp, f32, f32, f32,
                                          f32, vp]
    lib.dist_gemm_plan_steps.argtypes = [vp, ctypes.POINTER(Step), ctypes.POINTER(i32)]
    lib.dist_gemm_step_times.argtypes = [vp, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(i32)]
    lib.dist_gemm_step_timeline.argtypes = [vp, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(i32)]
    lib.dist_gemm_device_errors.argtypes = [vp, ctypes.POINTER(i64)]
    lib.dist_gemm_destroy.argtypes = [vp]
    lib.dist_gemm_last_error.argtypes = [vp]
    lib.dist_gemm_last_error.restype = ctypes.c_char_p
    lib.dist_gemm_status_string.argtypes = [i32]
    lib.dist_gemm_status_string.restype = ctypes.c_char_p
    for name in ("dist_gemm_step_table", "dist_gemm_fused_tables", "dist_gemm_plan", "dist_gemm_set_scales", "dist_gemm_set_result_scale",
                 "dist_gemm_set_bias",
                 "dist_gemm_set_option", "dist_gemm_run", "dist_gemm_run_ag", "dist_gemm_run_noalloc",
                 "dist_gemm_plan_steps",
                 "dist_gemm_step_times", "dist_gemm_step_timeline", "dist_gemm_device_errors",
                 "dist_gemm_destroy"):
        getattr(lib, name).restype = i32
    return lib


lib = _load()


def _check(rc: int, plan=None):
    if rc != 0:
        msg = lib.dist_gemm_last_error(plan)
        raise DistGemmError(rc, msg.decode() if msg else "")


def _enum(table, v):
    return table[v] if isinstance(v, str) else int(v)


def dist_gemm_step_table(M, N, K, L, TP, schedule, dtype) -> List[tuple]:
    n = ctypes.c_int(0)
    _check(lib.dist_gemm_step_table(M, N, K, L, TP, _enum(SCHEDULES, schedule),
                                    _enum(DTYPES, dtype), None, ctypes.byref(n)))
    arr = (Step * n.value)()
    _check(lib.dist_gemm_step_table(M, N, K, L, TP, _enum(SCHEDULES, schedule),
                                    _enum(DTYPES, dtype), arr, ctypes.byref(n)))
    return [s.as_tuple() for s in arr]


def dist_gemm_fused_tables(M, N, K, L, TP, schedule, dtype, shared_a=0, queues=8, step_group=2, copy_ahead=0,
                           copy_chunk=2 << 20, n_wg=256) -> dict:
    """The single launch's tables for these options (host only): the info
    fields, and the arrays segs [n_segs][4], steps [TP][7], strips
    [2 n_strips + TP], seg [queues][n_segs + 1] as lists of rows."""
    info = FusedInfo()
    args = (M, N, K, L, TP, _enum(SCHEDULES, schedule), _enum(DTYPES, dtype), shared_a, queues, step_group,
            copy_ahead, copy_chunk, n_wg)
    _check(lib.dist_gemm_fused_tables(*args, ctypes.byref(info), None, None, None, None))
    segs = (ctypes.c_int32 * (4 * info.n_segs))()
    steps = (ctypes.c_int64 * (7 * TP))()
    strips = (ctypes.c_int32 * (2 * info.n_strips + TP))()
    seg = (ctypes.c_int32 * (queues * (info.n_segs + 1)))()
    _check(lib.dist_gemm_fused_tables(*args, ctypes.byref(info), segs, steps, strips, seg))
    out = {name: getattr(info, name) for name, _ in FusedInfo._fields_ if name != "reserved"}
    out["segs"] = [list(segs[4 * g:4 * g + 4]) for g in range(info.n_segs)]
    out["steps"] = [list(steps[7 * h:7 * h + 7]) for h in range(TP)]
    out["strip_list"] = list(strips[:info.n_strips])
    out["strip_step"] = list(strips[info.n_strips:2 * info.n_strips])
    out["claim_steps"] = list(strips[2 * info.n_strips:])
    out["seg"] = [list(seg[q * (info.n_segs + 1):(q + 1) * (info.n_segs + 1)]) for q in range(queues)]
    return out


def dist_gemm_plan(M, N, K, L, TP, schedule, dtype) -> ctypes.c_void_p:
    h = ctypes.c_void_p()
    _check(lib.dist_gemm_plan(M, N, K, L, TP, _enum(SCHEDULES, schedule), _enum(DTYPES, dtype),
                              ctypes.byref(h)))
    return h


def dist_gemm_set_scales(plan, scale_a: float, scale_b: float):
    _check(lib.dist_gemm_set_scales(plan, scale_a, scale_b), plan)


def dist_gemm_set_result_scale(plan, scale_result: float):
    _check(lib.dist_gemm_set_result_scale(plan, scale_result), plan)


def dist_gemm_set_bias(plan, bias):
    _check(lib.dist_gemm_set_bias(plan, _ptr(bias)), plan)


def dist_gemm_set_option(plan, option, value: int):
    _check(lib.dist_gemm_set_option(plan, _enum(OPTIONS, option), int(value)), plan)


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream or None
    if isinstance(stream, int):
        return stream or None
    return stream.cuda_stream or None


def dist_gemm_run(plan, A, B, C, D, alpha: float = 1.0, beta: float = 0.0, stream=None):
    _check(lib.dist_gemm_run(plan, _ptr(A), _ptr(B), _ptr(C), _ptr(D), alpha, beta,
                             _stream(stream)), plan)


def dist_gemm_run_ag(plan, A, B, C, D, ag_out, alpha: float = 1.0, beta: float = 0.0, stream=None):
    _check(lib.dist_gemm_run_ag(plan, _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(ag_out), alpha, beta,
                                _stream(stream)), plan)


def dist_gemm_run_noalloc(M, N, K, L, TP, schedule, dtype, A, B, C, D, alpha: float = 1.0,
                          beta: float = 0.0, scale_a: float = 1.0, scale_b: float = 1.0, stream=None):
    _check(lib.dist_gemm_run_noalloc(M, N, K, L, TP, _enum(SCHEDULES, schedule), _enum(DTYPES, dtype),
                                     _ptr(A), _ptr(B), _ptr(C), _ptr(D), alpha, beta, scale_a, scale_b,
                                     _stream(stream)))


def dist_gemm_plan_steps(plan) -> List[tuple]:
    n = ctypes.c_int(0)
    _check(lib.dist_gemm_plan_steps(plan, None, ctypes.byref(n)), plan)
    arr = (Step * n.value)()
    _check(lib.dist_gemm_plan_steps(plan, arr, ctypes.byref(n)), plan)
    return [s.as_tuple() for s in arr]


def dist_gemm_step_times(plan) -> List[float]:
    n = ctypes.c_int(0)
    _check(lib.dist_gemm_step_times(plan, None, ctypes.byref(n)), plan)
    buf = (ctypes.c_float * max(n.value, 1))()
    _check(lib.dist_gemm_step_times(plan, buf, ctypes.byref(n)), plan)
    return [buf[i] for i in range(n.value)]


def dist_gemm_step_timeline(plan) -> List[tuple]:
    """(copy_done_ms or -1, begin_ms, end_ms) per step of the last timed run."""
    n = ctypes.c_int(0)
    _check(lib.dist_gemm_step_timeline(plan, None, ctypes.byref(n)), plan)
    buf = (ctypes.c_float * max(n.value, 1))()
    _check(lib.dist_gemm_step_timeline(plan, buf, ctypes.byref(n)), plan)
    return [tuple(buf[3 * s + k] for k in range(3)) for s in range(n.value // 3)]


def dist_gemm_device_errors(plan) -> int:
    """Timed-out device-side shard waits of the plan's single-launch runs so far."""
    n = ctypes.c_int64(0)
    _check(lib.dist_gemm_device_errors(plan, ctypes.byref(n)), plan)
    return n.value


def dist_gemm_destroy(plan):
    _check(lib.dist_gemm_destroy(plan))


class Plan:
    """Owning wrapper of a plan handle.  run() checks that tensor arguments
    are large enough and on a GPU before handing their addresses over."""

    def __init__(self, M, N, K, L=1, TP=1, schedule="MONOLITHIC", dtype="BF16_F32"):
        self.M, self.N, self.K, self.L, self.TP = M, N, K, L, TP
        self.schedule, self.dtype = schedule, dtype
        self.shared_a = False
        self.handle = dist_gemm_plan(M, N, K, L, TP, schedule, dtype)

    def set_scales(self, scale_a, scale_b):
        dist_gemm_set_scales(self.handle, scale_a, scale_b)

    def set_result_scale(self, scale_result):
        dist_gemm_set_result_scale(self.handle, scale_result)

    def set_bias(self, bias):
        """bias: a GPU tensor of N output elements (fp32, or bf16 bits), or None.
        The plan keeps its address; keep the tensor alive while runs may use it."""
        if bias is not None and not isinstance(bias, int):
            self._need(bias, self.N * ELEM_BYTES[self.dtype][1], "bias")
        self._bias = bias
        dist_gemm_set_bias(self.handle, bias)

    def set_option(self, option, value):
        dist_gemm_set_option(self.handle, option, value)
        if _enum(OPTIONS, option) == OPTIONS["SHARED_A"]:
            self.shared_a = bool(value)

    def steps(self):
        return dist_gemm_plan_steps(self.handle)

    def step_times(self):
        return dist_gemm_step_times(self.handle)

    def step_timeline(self):
        return dist_gemm_step_timeline(self.handle)

    def device_errors(self):
        return dist_gemm_device_errors(self.handle)

    def _need(self, t, nbytes, name):
        if t is None or isinstance(t, int):
            return
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.numel() * t.element_size() < nbytes:
            raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes, needs {nbytes}")

    def _check_operands(self, A, B, C, D):
        ei, eo = ELEM_BYTES[self.dtype]
        M, N, K, L = self.M, self.N, self.K, self.L
        self._need(A, (1 if self.shared_a else L) * M * K * ei, "A")
        self._need(B, L * N * K * ei, "B")
        self._need(D, L * M * N * eo, "D")
        if C is not None:
            self._need(C, L * M * N * eo, "C")

    def run(self, A, B, C, D, alpha=1.0, beta=0.0, stream=None):
        self._check_operands(A, B, C, D)
        dist_gemm_run(self.handle, A, B, C, D, alpha, beta, stream)

    def run_ag(self, A, B, C, D, ag_out, alpha=1.0, beta=0.0, stream=None):
        """run() that also writes the gathered rotating operand (A for AG_ROT_A,
        B for AG_ROT_B) into ag_out."""
        self._check_operands(A, B, C, D)
        ei = ELEM_BYTES[self.dtype][0]
        if _enum(SCHEDULES, self.schedule) == SCHEDULES["AG_ROT_A"]:
            self._need(ag_out, (1 if self.shared_a else self.L) * self.M * self.K * ei, "ag_out")
        else:
            self._need(ag_out, self.L * self.N * self.K * ei, "ag_out")
        dist_gemm_run_ag(self.handle, A, B, C, D, ag_out, alpha, beta, stream)

    def close(self):
        if self.handle is not None:
            dist_gemm_destroy(self.handle)
            self.handle = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
