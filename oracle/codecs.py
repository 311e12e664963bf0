"""Element codecs used by the oracle, written from the format definitions.

bf16  : the upper 16 bits of an IEEE-754 binary32 (1 sign, 8 exponent bits
        with bias 127, 7 mantissa bits).  Decoding is exact.
e4m3fn: OCP 8-bit float E4M3 ("fn": finite, no infinities).  1 sign bit,
        4 exponent bits with bias 7, 3 mantissa bits.  Exponent field 0 is
        subnormal (value m/8 * 2^-6); S.1111.111 is NaN; the largest finite
        magnitude is 1.75 * 2^8 = 448.  The scaled fp8 matmul of the PyTorch
        symmetric-memory page (fused_all_gather_scaled_matmul) multiplies the
        decoded values by per-tensor scales, which the oracle does in fp64.

Encoders round to nearest, ties to even, directly from float64 (no double
rounding through float32).  They are used by the oracle's own tests and for
rounding the fp64 result to the output element type.
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------- bf16

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def _round_to_grid(x: np.ndarray, mant_bits: int, emin: int) -> np.ndarray:
    """Round float64 x to the nearest value with `mant_bits` fraction bits and
    minimum normal exponent `emin` (subnormals below), ties to even.
    Overflow is not handled here."""
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    fin = np.isfinite(x) & (x != 0)
    xf = x[fin]
    _, e = np.frexp(xf)          # xf = f * 2^e, 0.5 <= |f| < 1  -> exponent e-1
    e = np.maximum(e - 1, emin)
    q = np.ldexp(1.0, e - mant_bits)  # spacing of the grid at that exponent
    out[fin] = np.rint(xf / q) * q    # xf/q is exact (power-of-two scaling); rint is RNE
    out[~np.isfinite(x)] = x[~np.isfinite(x)]
    out[x == 0] = x[x == 0]
    return out


BF16_MAX = float((2.0 - 2.0 ** -7) * 2.0 ** 127)


def f64_to_bf16_value(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bf16 value (RNE), returned as float64; overflow -> inf."""
    r = _round_to_grid(x, 7, -126)
    big = np.abs(r) > BF16_MAX
    r[big] = np.copysign(np.inf, r[big])
    return r


def f64_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round to bf16 (RNE) and return the 16-bit patterns."""
    v = f64_to_bf16_value(x).astype(np.float32)  # exact: v is representable in bf16
    bits = (v.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(np.asarray(x, dtype=np.float64))
    bits[nan] = np.uint16(0x7FC0)
    return bits

# ---------------------------------------------------------------- e4m3fn

E4M3_MAX = 448.0


def _e4m3_table() -> np.ndarray:
    t = np.empty(256, dtype=np.float64)
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            t[code] = np.nan
        elif e == 0:
            t[code] = s * (m / 8.0) * 2.0 ** (1 - 7)
        else:
            t[code] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return t


E4M3_TABLE = _e4m3_table()


def e4m3_to_f64(bits: np.ndarray) -> np.ndarray:
    return E4M3_TABLE[np.asarray(bits, dtype=np.uint8)]


_POS_CODES = np.array([c for c in range(0x7F)], dtype=np.uint8)   # 0x00..0x7E, ascending values
_POS_VALUES = E4M3_TABLE[:0x7F]


def f64_to_e4m3(x: np.ndarray, saturate: bool = True) -> np.ndarray:
    """Round to e4m3fn (RNE).  Beyond the largest finite value: saturate to
    +-448, or NaN (0x7F/0xFF) when saturate=False."""
    x = np.asarray(x, dtype=np.float64)
    r = _round_to_grid(x, 3, -6)
    over = np.abs(r) > E4M3_MAX
    mag = np.abs(r)
    mag = np.where(over, E4M3_MAX, mag)
    idx = np.searchsorted(_POS_VALUES, mag)        # exact hit: mag is on the grid
    idx = np.clip(idx, 0, 0x7E)
    codes = _POS_CODES[idx].copy()
    codes |= np.where(np.signbit(r), 0x80, 0).astype(np.uint8)
    nan = np.isnan(x) | (over & (not saturate))
    codes[nan] = np.where(np.signbit(x[nan]), 0xFF, 0x7F).astype(np.uint8)
    return codes

# ---------------------------------------------------------------- dispatch

def decode(arr: np.ndarray, elem: str) -> np.ndarray:
    if elem == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    if elem == "bf16":
        return bf16_to_f64(arr)
    if elem == "e4m3":
        return e4m3_to_f64(arr)
    raise ValueError(elem)


def round_to(x: np.ndarray, elem: str) -> np.ndarray:
    """Round an fp64 result to the output element, returned as float64 values."""
    if elem == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    if elem == "bf16":
        return f64_to_bf16_value(x)
    if elem == "e4m3":
        # the fp8 output cast saturates at +-448 (the largest finite e4m3fn)
        return e4m3_to_f64(f64_to_e4m3(x, saturate=True))
    raise ValueError(elem)
