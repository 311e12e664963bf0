"""Mutation check of the oracle's pins (CPU only).

Each case plants one plausible mistake in a temporary copy of the oracle
(a dropped term, a transposed or reversed operand, a wrong scale, a wrong
rotation or staging rule, a dropped or misindexed bias, a wrong exponent,
double rounding, a loosened or misindexed parity normaliser) and runs the
oracle's pin tests against that copy: every mutation must make them fail.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTATIONS = [
    ("oracle/gemm.py", "blk = blk + np.float64(beta) * Ch[l, st.m0:st.m1, st.n0:st.n1]", "blk = blk"),
    ("oracle/gemm.py", "b = Bh[l, st.n0:st.n1, :]", "b = Bh[l, st.n0:st.n1, ::-1]"),
    ("oracle/gemm.py", "Bh = codecs.decode(B, in_elem) * np.float64(scale_b)",
     "Bh = codecs.decode(B, in_elem) * np.float64(scale_a)"),
    ("oracle/gemm.py", "blk = np.float64(alpha) * acc\n", "blk = np.float64(alpha) * acc * (1 + 2.0 ** -40)\n"),
    ("oracle/schedule.py", "j = (rank + s) % S ", "j = (rank + s + 1) % S "),
    ("oracle/schedule.py", "out.append(Step(s, j, lo, hi, 0, N, s > 0))", "out.append(Step(s, j, lo, hi, 0, N, s > 1))"),
    ("oracle/gemm.py", "blk = blk + bh[st.n0:st.n1][None, :]", "blk = blk"),
    ("oracle/gemm.py", "blk = blk + bh[st.n0:st.n1][None, :]", "blk = blk + bh[st.n0:st.n1][::-1][None, :]"),
    ("oracle/gemm.py", "blk = blk + bh[ci][None, :]", "blk = blk + bh[ri % len(bh)][:, None]"),
    ("oracle/codecs.py", "t[code] = s * (m / 8.0) * 2.0 ** (1 - 7)", "t[code] = s * (m / 8.0) * 2.0 ** (0 - 7)"),
    ("oracle/codecs.py", "e = np.maximum(e - 1, emin)", "e = np.maximum(e, emin)"),
    ("oracle/codecs.py", "r = _round_to_grid(x, 7, -126)", "r = _round_to_grid(np.asarray(x, dtype=np.float32).astype(np.float64), 7, -126)"),
    # the parity metric's normaliser and bars
    ("oracle/parity.py", "den = den + abs(beta) * np.abs(C)", "den = den + beta * np.abs(C)"),
    ("oracle/parity.py", "den = den + abs(beta) * np.abs(C)", "den = den + 4 * abs(beta) * np.abs(C)"),
    ("oracle/parity.py", "den = den + abs(beta) * np.abs(C)", "den = den"),
    ("oracle/parity.py", "if beta != 0.0 and C is not None:", "if C is not None:"),
    ("oracle/parity.py", "den = den + np.abs(np.asarray(bias, dtype=np.float64))[None, :]", "den = den"),
    ("oracle/parity.py", "den = den + np.abs(np.asarray(bias, dtype=np.float64))[None, :]",
     "den = den + 4 * np.abs(np.asarray(bias, dtype=np.float64))[None, :]"),
    ("oracle/parity.py", "den = den + np.abs(np.asarray(bias, dtype=np.float64))[None, :]",
     "den = den + np.abs(np.asarray(bias, dtype=np.float64))[:, None]"),
    ("oracle/parity.py", "den = abs(alpha) * np.outer(row_norms, col_norms)", "den = alpha * np.outer(row_norms, col_norms)"),
    ("oracle/parity.py", "tight = bool(np.all(diff <= 2.0 ** -8 * np.abs(ref) + t * den))",
     "tight = bool(np.all(diff <= 2.0 ** -7 * np.abs(ref) + t * den))"),
    # the result scale of an fp8 output, and the e4m3 output cast
    ("oracle/gemm.py", "D[l, st.m0:st.m1, st.n0:st.n1] = np.float64(result_scale) * blk",
     "D[l, st.m0:st.m1, st.n0:st.n1] = blk"),
    ("oracle/parity.py", "return abs(result_scale) * den", "return den"),
    ("oracle/parity.py", "return abs(result_scale) * den", "return result_scale * den"),
    ("oracle/parity.py", "return np.clip(D_star, -codecs.E4M3_MAX, codecs.E4M3_MAX)", "return D_star"),
    ("oracle/parity.py", "tight = bool(np.all(diff <= 2.0 ** -4 * np.abs(ref) + 2.0 ** -10 + t * den))",
     "tight = bool(np.all(diff <= 2.0 ** -3 * np.abs(ref) + 2.0 ** -10 + t * den))"),
    ("oracle/parity.py", "tight = bool(np.all(diff <= 2.0 ** -4 * np.abs(ref) + 2.0 ** -10 + t * den))",
     "tight = bool(np.all(diff <= 2.0 ** -4 * np.abs(ref) + 2.0 ** -9 + t * den))"),
    ("oracle/codecs.py", "return e4m3_to_f64(f64_to_e4m3(x, saturate=True))", "return e4m3_to_f64(f64_to_e4m3(x, saturate=False))"),
]


PIN_TESTS = ("test_oracle_codecs.py", "test_oracle_gemm.py", "test_oracle_parity_and_inputs.py")


@pytest.mark.parametrize("idx", range(len(MUTATIONS)))
def test_pins_catch_planted_mistake(idx, tmp_path):
    f, old, new = MUTATIONS[idx]
    for d in ("oracle", "workloads"):
        shutil.copytree(os.path.join(ROOT, d), tmp_path / d,
                        ignore=shutil.ignore_patterns("__pycache__"))
    (tmp_path / "tests").mkdir()
    for t in PIN_TESTS + ("conftest.py",):
        shutil.copy(os.path.join(ROOT, "tests", t), tmp_path / "tests" / t)
    src = (tmp_path / f).read_text()
    assert old in src, f"mutation anchor not found in {f}"
    (tmp_path / f).write_text(src.replace(old, new, 1))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        *[f"tests/{t}" for t in PIN_TESTS]],
                       cwd=tmp_path, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"pins did not catch mutation {idx}: {new!r}\n{r.stdout[-2000:]}"
