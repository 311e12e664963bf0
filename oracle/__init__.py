"""CPU oracle for the TP-step GEMM  D = alpha * A * B + beta * C.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: only the tests, the package's smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code with the HIP library
(no kernels, headers, tables or helpers); the only thing both sides consume
is the seeded operand bytes drawn by ``workloads``.

What it computes (plain, slow, fp64):
  * codecs.py   -- bf16 and OCP e4m3fn decoders/encoders written from the
                   format definitions;
  * schedule.py -- the per-step table of the four TP schedules named on the
                   CUTLASS Distributed GEMM example page ("Trying out other
                   schedules") plus the single-step monolithic GEMM;
  * gemm.py     -- the step-by-step fp64 GEMM with the alpha/beta epilogue,
                   one numpy float64 matmul per step;
  * parity.py   -- the per-element error normalised by row/column norms.

Every function is pinned by the CPU tests (brute force in exact rational
arithmetic, closed forms, schedule invariants, exhaustive codec tables,
the shapes and rates printed on the Distributed GEMM pull-request page,
and the output mean printed on the chunked all_gather+matmul blog page).
"""
from . import codecs, schedule, gemm, parity  # noqa: F401
