"""CPU checks of the parity metric and of the seeded input generator."""
import numpy as np
import pytest

import workloads
from oracle import codecs, gemm, parity


def test_metric_flags_planted_errors():
    g = np.random.default_rng(2)
    Dstar = g.standard_normal((8, 8))
    rn = np.ones(8)
    cn = np.ones(8)
    good = Dstar + 1e-7
    ok, mx, tight, _ = parity.check(good, Dstar, rn, cn, 1.0, 0.0, None, "f32", "f32")
    assert ok and tight and mx < 2e-7
    bad = Dstar.copy()
    bad[3, 4] += 1e-3
    ok, mx, tight, _ = parity.check(bad, Dstar, rn, cn, 1.0, 0.0, None, "f32", "f32")
    assert not ok and not tight
    nan = Dstar.copy()
    nan[0, 0] = np.nan
    assert not parity.check(nan, Dstar, rn, cn, 1.0, 0.0, None, "bf16", "bf16")[0]


def test_metric_zero_normaliser_needs_exact_value():
    Dstar = np.zeros((2, 2))
    z = np.zeros(2)
    assert parity.check(np.zeros((2, 2)), Dstar, z, z, 1.0, 0.0, None, "f32", "f32")[0]
    assert not parity.check(np.full((2, 2), 1e-30), Dstar, z, z, 1.0, 0.0, None, "f32", "f32")[0]


def test_bf16_output_rounding_passes_tight_bar():
    g = np.random.default_rng(3)
    Dstar = g.standard_normal((64, 64)) * 10
    dev = codecs.round_to(Dstar, "bf16")
    rn = np.full(64, 3.0)
    ok, mx, tight, _ = parity.check(dev, Dstar, rn, rn, 1.0, 0.0, None, "e4m3", "bf16")
    assert ok and tight
    # one ulp off somewhere fails the tight bar
    dev2 = dev.copy()
    dev2[5, 5] = Dstar[5, 5] * (1 + 2.0 ** -6)
    assert not parity.check(dev2, Dstar, rn, rn, 1.0, 0.0, None, "e4m3", "bf16")[2]


def test_generator_is_deterministic_and_shaped():
    for name in ("c1_tiny_ag_rot_a_f32",):
        w = workloads.CONFIGS[name]
        x1 = workloads.generate(w, need_c=True)
        x2 = workloads.generate(w, need_c=True)
        assert x1.A.shape == (1, 256, 256) and x1.B.shape == (1, 256, 256) and x1.C.shape == (1, 256, 256)
        assert np.array_equal(x1.A, x2.A) and np.array_equal(x1.C, x2.C)
        assert x1.A.min() >= -1 and x1.A.max() < 1


def test_generator_bf16_and_e4m3_encodings():
    w = workloads.small_case("b", "AG_ROT_A", "BF16_F32", 64, 32, 256)
    x = workloads.generate(w)
    assert x.A.dtype == np.uint16 and x.C is None
    a = codecs.bf16_to_f64(x.A)
    assert 0.5 / 16 < a.std() < 2 / 16
    w8 = workloads.small_case("e", "AG_ROT_B", "E4M3_BF16", 64, 32, 256)
    x8 = workloads.generate(w8)
    assert x8.A.dtype == np.uint8
    v = codecs.e4m3_to_f64(x8.A)
    assert np.max(np.abs(v)) == 448.0          # amax maps to the largest finite code
    assert not np.any(np.isnan(v))
    assert 0 < x8.scale_a < 1


def test_config_table():
    c = workloads.CONFIGS
    assert [w.name[:2] for w in c.values()] == ["c1", "c2", "c3", "c4", "c5"]
    c3 = c["c3_ag_rot_a_bf16_tp8"]
    assert (c3.M, c3.N, c3.K, c3.TP) == (16384, 13312, 16384, 8)
    assert c3.flops == 2.0 * 16384 * 13312 * 16384
    assert c["c4_rs_tile_a_rot_c_bf16_tp8"].beta == 1.0
    assert c["c5_ag_rot_b_e4m3_tp8"].out_dtype == "bf16"
