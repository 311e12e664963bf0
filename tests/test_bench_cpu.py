"""CPU tests of bench.py's host logic: the kernel-source hash that keys the
recorded HBM traffic, and the one-GPU contract of the command line."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.fixture
def source_copy(tmp_path, monkeypatch):
    for f in bench.KERNEL_SOURCES:
        dst = tmp_path / f
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(os.path.join(ROOT, f), dst)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    return tmp_path


def test_source_hash_ignores_comments_and_blank_lines(source_copy):
    h0 = bench.kernel_source_hash()
    p = source_copy / bench.KERNEL_SOURCES[1]
    text = p.read_text()
    p.write_text("// a comment line\n\n/* a block\n   comment */\n" + text.replace(";\n", ";  // trailing\n", 3))
    assert bench.kernel_source_hash() == h0


def test_source_hash_sees_code_changes(source_copy):
    h0 = bench.kernel_source_hash()
    p = source_copy / bench.KERNEL_SOURCES[2]
    p.write_text(p.read_text().replace("constexpr int kBM = 256;", "constexpr int kBM = 128;"))
    assert bench.kernel_source_hash() != h0


def test_traffic_record_is_keyed_by_the_hash(source_copy, monkeypatch):
    # the committed record, read against a changed code base, reports nothing
    rec = os.path.join(ROOT, bench.TRAFFIC_FILE)
    (source_copy / bench.TRAFFIC_FILE).parent.mkdir(parents=True, exist_ok=True)
    shutil.copy(rec, source_copy / bench.TRAFFIC_FILE)
    p = source_copy / bench.KERNEL_SOURCES[0]
    p.write_text(p.read_text() + "\nint traffic_record_probe_symbol;\n")
    assert bench.recorded_traffic("c3_ag_rot_a_bf16_tp8") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
