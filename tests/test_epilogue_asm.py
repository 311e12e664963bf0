"""The fp32 epilogue with C streams C into LDS with buffer_load ... lds and
waits for each 16-row part with s_waitcnt vmcnt immediates derived from its
own issue order (C loads and D stores share the counter and retire in order).
Those immediates are only right if the compiler puts no other vector-memory
instruction (a register spill, a reload) between a C load and its wait.  This
test compiles the GEMM units to gfx950 assembly with the library's flags and
checks, in every kernel that has the epilogue, that its vector-memory
instructions from the first C load on are exactly the designed sequence.

CPU only (hipcc cross-compiles); skipped where hipcc is missing.
"""
import importlib.util
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PARTS, AHEAD, PER_PART = 8, 2, 8  # 16-row parts, parts in flight, instructions per part


def _build_module():
    spec = importlib.util.spec_from_file_location(
        "_distgemm_build_cfg", os.path.join(ROOT, "communication_tensor_gemm_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _device_asm(B, src, out):
    cmd = [B.hipcc(), *B.HIPCC_FLAGS, *B.EXTRA.get(src, []), "--cuda-device-only", "-S",
           os.path.join(B.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return open(out).read()


def _kernels(text):
    funcs, name = {}, None
    for line in text.splitlines():
        m = re.match(r"^(_Z\S+):", line)
        if m:
            name = m.group(1)
            funcs[name] = []
            continue
        if name:
            funcs[name].append(line)
    return funcs


def _expected():
    seq = ["C"] * (AHEAD * PER_PART)
    for p in range(PARTS):
        if p + AHEAD < PARTS:
            seq += ["C"] * PER_PART
        seq += ["S"] * PER_PART
    return seq


def _vm_sequence(body):
    """Vector-memory instructions after the last MFMA, from the first LDS DMA
    on: 'C' for a C load into LDS, 'S' for a 16-byte global store, else the
    mnemonic; cut once all the epilogue's stores have been seen."""
    last_mfma = max(i for i, l in enumerate(body) if "v_mfma" in l)
    seq, started = [], False
    want_stores = PARTS * PER_PART
    for line in body[last_mfma:]:
        tok = line.split()
        if not tok or tok[0].startswith((";", ".")):
            continue
        op = tok[0]
        if "offen lds" in line:
            started = True
            seq.append("C")
        elif not started:
            continue
        elif op == "global_store_dwordx4":
            seq.append("S")
        elif op.startswith(("global_", "buffer_", "flat_", "scratch_")):
            seq.append(op)
        if seq.count("S") == want_stores:
            break
    return seq


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_c_epilogue_memory_sequence(tmp_path):
    B = _build_module()
    srcs = ["gemm_mfma16.hip", "gemm_mfma_f8.hip"]
    with ThreadPoolExecutor(2) as ex:
        texts = list(ex.map(lambda s: _device_asm(B, s, str(tmp_path / (s + ".s"))), srcs))
    expected = _expected()
    checked = []
    for text in texts:
        for name, body in _kernels(text).items():
            if not any("v_mfma" in l for l in body):
                continue
            last_mfma = max(i for i, l in enumerate(body) if "v_mfma" in l)
            if not any("offen lds" in l for l in body[last_mfma:]):
                continue  # no C epilogue in this kernel (bf16 output)
            seq = _vm_sequence(body)
            assert seq == expected, (name, seq[:80])
            checked.append(name)
    # fp32 output: bf16 / fp32 / e4m3 inputs, per-step and persistent kernels
    assert len(checked) == 6, checked
