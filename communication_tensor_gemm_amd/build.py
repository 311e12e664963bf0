"""Build libdistgemm.so for gfx950 with hipcc (in-tree, no JIT cache).

    python communication_tensor_gemm_amd/build.py

(By path: importing the package needs the library this builds.)
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libdistgemm.so")
BUILD_DIR = os.path.join(ROOT, "_build")
SOURCES = ["gemm_mfma16.hip", "gemm_mfma_f8.hip", "distgemm.hip"]
# per-source extra flags
EXTRA = {
    # the fp32 half slab is 256 MFMAs long; without a higher threshold the
    # unroller gives up and the accumulators become a stack array
    "gemm_mfma16.hip": ["-mllvm", "-pragma-unroll-threshold=1000000"],
    # same guard for the fp8 unit's fully unrolled slab and epilogue
    "gemm_mfma_f8.hip": ["-mllvm", "-pragma-unroll-threshold=1000000"],
}
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # packed fp32 arithmetic stays off (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "argument unused during compilation: '--hip-link'"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if noise not in l and "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{msg}")
    if verbose and msg:
        print(msg)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([cc, *HIPCC_FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = OUT + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
