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


# ---- the beta*|C|, |alpha| and |bias| terms of the normaliser ---------------
#
# Each case builds operands whose norms make one term dominate the
# normaliser, plants one element error at a known multiple of the f32 bar
# times the true normaliser of that element, and checks both sides of the
# bar: 0.3 x bar must pass and 3 x bar must fail.  A dropped term shrinks
# the normaliser (the 0.3 x case then fails), an inflated one grows it (the
# 3 x case then passes), and a dropped abs() makes it non-positive for a
# negative scalar (the 0.3 x case then needs an exact value and fails).

def _true_den(rn, cn, alpha, beta, C, bias):
    """The normaliser written out element by element from its definition."""
    den = np.empty((len(rn), len(cn)))
    for i in range(len(rn)):
        for j in range(len(cn)):
            v = abs(alpha) * rn[i] * cn[j]
            if beta != 0.0:
                v += abs(beta) * abs(C[i, j])
            if bias is not None:
                v += abs(bias[j])
            den[i, j] = v
    return den


def _plant(alpha, beta, C, bias, rn, cn, factor, at=(2, 3)):
    g = np.random.default_rng(11)
    Dstar = g.standard_normal((len(rn), len(cn)))
    den = _true_den(rn, cn, alpha, beta, C, bias)
    dev = Dstar.copy()
    dev[at] += factor * parity.BARS["f32"] * den[at]
    return parity.check(dev, Dstar, rn, cn, alpha, beta, C, "f32", "f32", bias)


@pytest.mark.parametrize("beta", [1.0, -0.5])
def test_metric_c_term_scales_the_bar(beta):
    # tiny operand norms: the normaliser is |beta| * |C| almost everywhere
    rn = np.full(6, 1e-4)
    cn = np.full(5, 1e-4)
    C = np.random.default_rng(5).uniform(50.0, 100.0, (6, 5)) * np.where(
        np.arange(30).reshape(6, 5) % 2 == 0, 1.0, -1.0)
    ok, mx, _, _ = _plant(1.0, beta, C, None, rn, cn, 0.3)
    assert ok and 0.25 * parity.BARS["f32"] < mx < 0.35 * parity.BARS["f32"]
    ok, mx, _, _ = _plant(1.0, beta, C, None, rn, cn, 3.0)
    assert not ok and 2.9 * parity.BARS["f32"] < mx < 3.1 * parity.BARS["f32"]


def test_metric_c_term_ignored_when_beta_is_zero():
    # beta = 0: C is not part of the result, so it must not loosen the bar
    rn = np.full(6, 1e-4)
    cn = np.full(5, 1e-4)
    C = np.full((6, 5), 1e6)
    ok, _, _, _ = _plant(1.0, 0.0, C, None, rn, cn, 3.0)
    assert not ok
    # nor can a non-finite C that is never read spoil a correct result
    C[1, 1] = np.inf
    C[2, 2] = np.nan
    ok, mx, tight, _ = _plant(1.0, 0.0, C, None, rn, cn, 0.3)
    assert ok and tight and np.isfinite(mx)


@pytest.mark.parametrize("alpha", [2.0, -2.0])
def test_metric_alpha_term_scales_the_bar(alpha):
    rn = np.random.default_rng(6).uniform(1.0, 3.0, 6)
    cn = np.random.default_rng(7).uniform(1.0, 3.0, 5)
    assert _plant(alpha, 0.0, None, None, rn, cn, 0.3)[0]
    assert not _plant(alpha, 0.0, None, None, rn, cn, 3.0)[0]


def test_metric_bias_term_scales_the_bar():
    rn = np.full(6, 1e-4)
    cn = np.full(5, 1e-4)
    bias = np.array([40.0, -60.0, 80.0, -90.0, 70.0])
    for at in [(2, 3), (0, 1), (5, 4)]:
        ok, mx, _, _ = _plant(1.0, 0.0, None, bias, rn, cn, 0.3, at)
        assert ok and mx > 0.25 * parity.BARS["f32"]
        assert not _plant(1.0, 0.0, None, bias, rn, cn, 3.0, at)[0]


def test_metric_bias_and_c_terms_add():
    rn = np.full(6, 1e-4)
    cn = np.full(5, 1e-4)
    C = np.full((6, 5), -30.0)
    bias = np.full(5, 30.0)
    # both terms count: 0.6 x the bar measured against |C| alone passes only
    # because the bias term doubles the normaliser
    ok, mx, _, _ = _plant(1.0, -1.0, C, bias, rn, cn, 0.3)
    assert ok and 0.25 * parity.BARS["f32"] < mx < 0.35 * parity.BARS["f32"]
    assert not _plant(1.0, -1.0, C, bias, rn, cn, 3.0)[0]


def test_bf16_output_tight_bar_is_half_an_ulp_of_rounding():
    # the tight bf16-output bar allows 2^-8 |D*| (round to nearest), not more
    g = np.random.default_rng(4)
    Dstar = g.uniform(1.0, 2.0, (32, 32)) * np.where(g.random((32, 32)) < 0.5, -1.0, 1.0)
    rn = np.full(32, 1e-3)
    dev = Dstar * (1 + 0.9 * 2.0 ** -8)
    assert parity.check(dev, Dstar, rn, rn, 1.0, 0.0, None, "bf16", "bf16")[2]
    dev = Dstar.copy()
    dev[7, 9] = Dstar[7, 9] * (1 + 1.5 * 2.0 ** -8)
    assert not parity.check(dev, Dstar, rn, rn, 1.0, 0.0, None, "bf16", "bf16")[2]


@pytest.mark.parametrize("s", [2.5, -4.0])
def test_metric_result_scale_scales_the_bar(s):
    """The result scale multiplies the whole result, so its magnitude scales
    the normaliser; planted errors on both sides of the bar."""
    rn = np.random.default_rng(6).uniform(1.0, 3.0, 6)
    cn = np.random.default_rng(7).uniform(1.0, 3.0, 5)
    g = np.random.default_rng(8)
    Dstar = g.standard_normal((6, 5))
    for factor, want in ((0.3, True), (3.0, False)):
        dev = Dstar.copy()
        den = abs(s) * 2.0 * rn[2] * cn[3]
        dev[2, 3] += factor * parity.BARS["f32"] * den
        assert parity.check(dev, Dstar, rn, cn, 2.0, 0.0, None, "f32", "f32", None, s)[0] == want


def test_e4m3_output_bars():
    """e4m3 output: the cast saturates at 448 (a saturated result is exact);
    the tight bar is half a spacing of three mantissa bits (2^-4 relative,
    2^-10 absolute below 2^-6), no more."""
    rn = np.full(4, 1e-3)
    # 100 -> 104: half a spacing (8); 6.5 * 2^-9 -> 6 * 2^-9: half the subnormal spacing
    Dstar = np.array([[500.0, -1000.0, 100.0, 6.5 * 2.0 ** -9]] * 4)
    dev = np.array([[448.0, -448.0, 104.0, 6.0 * 2.0 ** -9]] * 4)
    ok, mx, tight, _ = parity.check(dev, Dstar, rn, rn, 1.0, 0.0, None, "e4m3", "e4m3")
    assert tight
    bad = dev.copy()
    bad[1, 0] = 416.0           # one spacing below the saturated value
    assert not parity.check(bad, Dstar, rn, rn, 1.0, 0.0, None, "e4m3", "e4m3")[2]
    bad = dev.copy()
    bad[2, 2] = 112.0           # a full spacing off 100
    assert not parity.check(bad, Dstar, rn, rn, 1.0, 0.0, None, "e4m3", "e4m3")[2]
    bad = dev.copy()
    bad[3, 3] = 7.7 * 2.0 ** -9  # subnormal region: 1.2 * 2^-9 off, beyond half the spacing
    assert not parity.check(bad, Dstar, rn, rn, 1.0, 0.0, None, "e4m3", "e4m3")[2]
