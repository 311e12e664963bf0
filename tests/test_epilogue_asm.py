"""The fp32 epilogue with C streams C into LDS with buffer_load ... lds and
waits for each 16-row part with s_waitcnt vmcnt immediates derived from its
own issue order (C loads and D stores share the counter and retire in order).
A wait vmcnt(N) covers a C load once at least N vector-memory operations
were issued after it, so the immediates are right as long as the compiler
issues exactly the designed loads and stores, in that order: a missing or
moved one would let a wait pass early.  An extra one (a register spill or
reload) only makes a wait stricter.  This test compiles the GEMM units to
gfx950 assembly with the library's flags and checks, in every kernel that
has the epilogue, that its global and buffer memory instructions contain
the designed sequence with nothing else in between (scratch spills and
reloads, if any, are reported and allowed).

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
    """The kernel's vector-memory instructions in program order: 'C' for a
    load into LDS, 'S' for a 16-byte global store, else the mnemonic.  (The
    persistent kernels' shard-copy loop loads into LDS too.)"""
    seq = []
    for line in body:
        tok = line.split()
        if not tok or tok[0].startswith((";", ".")):
            continue
        op = tok[0]
        if "offen lds" in line:
            seq.append("C")
        elif op == "global_store_dwordx4":
            seq.append("S")
        elif op.startswith(("global_", "buffer_", "flat_", "scratch_")):
            seq.append(op)
    return seq


def _contains(seq, pattern):
    n = len(pattern)
    return any(seq[i:i + n] == pattern for i in range(len(seq) - n + 1))


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
            m = re.search(r"ILi(\d+)ELi(\d+)EEEv", name)
            if not m or int(m.group(2)) != 0 or not any("v_mfma" in l for l in body):
                continue  # the C epilogue belongs to the fp32-output kernels
            seq = _vm_sequence(body)
            spills = [op for op in seq if op.startswith("scratch_")]
            seq = [op for op in seq if not op.startswith("scratch_")]
            # the designed sequence, with no other global or buffer access in between
            assert _contains(seq, expected), (name, seq[:160])
            if spills:
                print(f"{name}: {len(spills)} scratch accesses (allowed)")
            checked.append(name)
    # fp32 output: bf16 / fp32 / e4m3 inputs, per-step and persistent kernels
    assert len(checked) == 6, checked
