"""Per-element error of a device result against the oracle.

err_ij = |D~_ij - D*_ij| / ( |s| * (|alpha| * ||Ahat_i,:||_2 * ||Bhat_:,j||_2 + |beta| * |C_ij| + |bias_j|) )

D* is the unrounded fp64 oracle value and Ahat/Bhat the decoded, scaled
operands; s is the result scale of an fp8 output (1 otherwise).  For an e4m3
output, whose cast saturates at +-448, D* is clipped to [-448, 448] first
(the saturation belongs to the cast).  The normaliser bounds |D*_ij| (Cauchy-Schwarz), so the error is
relative to the size the dot product could have, not to a possibly cancelled
result.  Where the normaliser is 0 the device value must equal D* rounded to
the output element.  Any NaN in the device result fails.

Bars: fp32 inputs 1e-5, bf16 inputs 2e-2, e4m3 inputs 6e-2 (max over
elements).  Tighter regression bars, which reflect that both sides consume
the same operand bytes so only the accumulation and the final rounding
differ:
  * fp32 output   : err <= t
  * bf16 output   : |D~ - D*| <= 2^-8 |D*| + t * normaliser
  * e4m3 output   : |D~ - D*| <= 2^-4 |D*| + 2^-10 + t * normaliser (half a
                    spacing of three mantissa bits; 2^-10 below 2^-6, where
                    the spacing is 2^-9)
with t = 1e-5 for fp32 and bf16 inputs (fp32 accumulation) and t = 1e-4 for
e4m3 inputs, whose 64-product MFMA reduction rounds internally more coarsely
than an fp32 sum (measured normalised errors up to 1.2e-5 at K = 128,
falling with K; fp32 and bf16 inputs stay below 3e-7).
"""
from __future__ import annotations

import numpy as np

from . import codecs

BARS = {"f32": 1e-5, "bf16": 2e-2, "e4m3": 6e-2}
TIGHT_ACCUM = {"f32": 1e-5, "bf16": 1e-5, "e4m3": 1e-4}


def normaliser(row_norms, col_norms, alpha: float, beta: float, C=None, bias=None,
               result_scale: float = 1.0):
    """bias: the decoded bias values of the compared columns (or None)."""
    den = abs(alpha) * np.outer(row_norms, col_norms)
    if beta != 0.0 and C is not None:
        den = den + abs(beta) * np.abs(C)
    if bias is not None:
        den = den + np.abs(np.asarray(bias, dtype=np.float64))[None, :]
    return abs(result_scale) * den


def _reference(D_star, out_elem: str):
    if out_elem == "e4m3":
        return np.clip(D_star, -codecs.E4M3_MAX, codecs.E4M3_MAX)
    return D_star


def normalised_error(D_dev, D_star, row_norms, col_norms, alpha: float, beta: float, C=None,
                     out_elem: str = "f32", bias=None, result_scale: float = 1.0):
    """Returns the per-element error array (inf where it fails outright)."""
    D_dev = np.asarray(D_dev, dtype=np.float64)
    den = normaliser(row_norms, col_norms, alpha, beta, C, bias, result_scale)
    D_star = _reference(np.asarray(D_star, dtype=np.float64), out_elem)
    diff = np.abs(D_dev - D_star)
    err = np.zeros_like(diff)
    pos = den > 0
    err[pos] = diff[pos] / den[pos]
    zero = ~pos
    if zero.any():
        exact = codecs.round_to(D_star[zero], out_elem)
        err[zero] = np.where(D_dev[zero] == exact, 0.0, np.inf)
    err[np.isnan(D_dev)] = np.inf
    return err


def check(D_dev, D_star, row_norms, col_norms, alpha, beta, C, in_elem: str, out_elem: str,
          bias=None, result_scale: float = 1.0):
    """(ok, max_err, tight_ok, detail) under the bar of the input element and the
    tight output-rounding bar.  bias: decoded bias of the compared columns."""
    err = normalised_error(D_dev, D_star, row_norms, col_norms, alpha, beta, C, out_elem, bias,
                           result_scale)
    mx = float(err.max()) if err.size else 0.0
    ok = mx <= BARS[in_elem]
    den = normaliser(row_norms, col_norms, alpha, beta, C, bias, result_scale)
    ref = _reference(np.asarray(D_star, dtype=np.float64), out_elem)
    diff = np.abs(np.asarray(D_dev, dtype=np.float64) - ref)
    t = TIGHT_ACCUM[in_elem]
    if out_elem == "f32":
        tight = bool(np.all(err <= t))
    elif out_elem == "bf16":
        tight = bool(np.all(diff <= 2.0 ** -8 * np.abs(ref) + t * den))
    else:
        tight = bool(np.all(diff <= 2.0 ** -4 * np.abs(ref) + 2.0 ** -10 + t * den))
    return ok, mx, tight, {"max_err": mx, "n": int(err.size)}
