"""Pins for the oracle's element codecs (CPU only).

The decoders and encoders are checked against the format definitions
(hand-listed code points, monotonicity, round trips, ties-to-even at every
midpoint) and against PyTorch's own CPU casts, which are an independent
implementation of the same formats.
"""
import numpy as np
import pytest
import torch

from oracle import codecs


# ------------------------------------------------------------------ e4m3fn

KNOWN_E4M3 = {
    0x00: 0.0,
    0x01: 2.0 ** -9,            # smallest subnormal
    0x07: 7 * 2.0 ** -9,        # largest subnormal
    0x08: 2.0 ** -6,            # smallest normal
    0x30: 0.5,
    0x38: 1.0,
    0x39: 1.125,
    0x3C: 1.5,
    0x40: 2.0,
    0x77: 240.0,
    0x78: 256.0,
    0x7E: 448.0,                # largest finite
    0xB8: -1.0,
    0xFE: -448.0,
}


def test_e4m3_known_points():
    for code, val in KNOWN_E4M3.items():
        assert codecs.e4m3_to_f64(np.uint8(code)) == val, hex(code)
    assert np.isnan(codecs.e4m3_to_f64(np.uint8(0x7F)))
    assert np.isnan(codecs.e4m3_to_f64(np.uint8(0xFF)))
    neg0 = codecs.e4m3_to_f64(np.uint8(0x80))
    assert neg0 == 0.0 and np.signbit(neg0)


def test_e4m3_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = codecs.e4m3_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    both_nan = np.isnan(ours) & np.isnan(ref)
    assert np.all(both_nan | (ours == ref))
    assert np.array_equal(np.signbit(ours[~both_nan]), np.signbit(ref[~both_nan]))
    assert int(np.isnan(ours).sum()) == 2


def test_e4m3_positive_codes_strictly_increase():
    v = codecs.e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(v) > 0)


def test_e4m3_round_trip_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    back = codecs.f64_to_e4m3(codecs.e4m3_to_f64(codes))
    assert np.array_equal(back, codes)


def test_e4m3_ties_to_even_at_every_midpoint():
    pos = codecs.e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2.0
    got = codecs.f64_to_e4m3(mids)
    lo = np.arange(0x7E, dtype=np.uint8)
    expect = np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint8)
    assert np.array_equal(got, expect)
    assert np.array_equal(codecs.f64_to_e4m3(-mids), expect | 0x80)
    # just off the midpoint goes to the nearer neighbour
    eps = np.diff(pos) * 1e-6
    assert np.array_equal(codecs.f64_to_e4m3(mids - eps), lo)
    assert np.array_equal(codecs.f64_to_e4m3(mids + eps), lo + 1)


def test_e4m3_saturation_and_nan():
    assert codecs.f64_to_e4m3(np.array([1000.0]))[0] == 0x7E
    assert codecs.f64_to_e4m3(np.array([-1000.0]))[0] == 0xFE
    assert codecs.f64_to_e4m3(np.array([1000.0]), saturate=False)[0] == 0x7F
    assert codecs.f64_to_e4m3(np.array([464.0]))[0] == 0x7E   # tie between 448 and 480 -> even
    assert codecs.f64_to_e4m3(np.array([np.nan]))[0] == 0x7F


def test_e4m3_encode_matches_torch_on_random_values():
    g = np.random.default_rng(5)
    x = np.concatenate([
        g.standard_normal(20000) * 50,
        g.standard_normal(5000) * 2.0 ** -8,     # subnormal range
        g.uniform(-448, 448, 5000),
    ]).astype(np.float32)
    ours = codecs.f64_to_e4m3(x.astype(np.float64))
    ref = torch.from_numpy(x).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


# ------------------------------------------------------------------ bf16

def test_bf16_decode_all_patterns_match_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = codecs.bf16_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    both_nan = np.isnan(ours) & np.isnan(ref)
    assert np.all(both_nan | (ours == ref))


def test_bf16_known_points():
    assert codecs.bf16_to_f64(np.uint16(0x3F80)) == 1.0
    assert codecs.bf16_to_f64(np.uint16(0xC000)) == -2.0
    assert codecs.bf16_to_f64(np.uint16(0x0001)) == 2.0 ** -133     # smallest subnormal
    assert codecs.bf16_to_f64(np.uint16(0x7F7F)) == codecs.BF16_MAX
    assert np.isinf(codecs.bf16_to_f64(np.uint16(0x7F80)))


def test_bf16_ties_to_even_and_subnormals():
    # 1 + 2^-8 is the midpoint of 1 and 1 + 2^-7 -> even (1.0)
    assert codecs.f64_to_bf16(np.array([1.0 + 2.0 ** -8]))[0] == 0x3F80
    # 1 + 3*2^-8 is the midpoint of 1+2^-7 and 1+2^-6 -> even (1 + 2^-6)
    assert codecs.f64_to_bf16(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 0x3F82
    # a value just above a midpoint, below float32 resolution of the midpoint:
    # fp64 -> bf16 directly must not double-round through fp32
    x = 1.0 + 2.0 ** -8 + 2.0 ** -40
    assert codecs.f64_to_bf16(np.array([x]))[0] == 0x3F81
    assert codecs.f64_to_bf16(np.array([2.0 ** -134]))[0] == 0x0000    # tie -> even (0)
    assert codecs.f64_to_bf16(np.array([3 * 2.0 ** -134]))[0] == 0x0002
    assert codecs.f64_to_bf16(np.array([1e39]))[0] == 0x7F80            # overflow -> inf


def test_bf16_encode_matches_torch_on_float32_inputs():
    g = np.random.default_rng(6)
    x = np.concatenate([
        g.standard_normal(50000).astype(np.float32),
        (g.standard_normal(5000) * 1e-39).astype(np.float32),          # subnormals
        g.integers(0, 2 ** 32, 20000, dtype=np.uint64).astype(np.uint32).view(np.float32),
    ])
    x = x[np.isfinite(x)]
    ours = codecs.f64_to_bf16(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_round_to_f32_is_rne():
    x = np.array([1.0 + 2.0 ** -24, 1.0 + 3 * 2.0 ** -24])
    r = codecs.round_to(x, "f32")
    assert r[0] == 1.0 and r[1] == 1.0 + 2.0 ** -22
