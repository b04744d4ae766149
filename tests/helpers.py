"""Test-only helpers: tensor <-> numpy marshalling for the oracle and the
comparison rules used by the parity tests."""

from __future__ import annotations

import numpy as np
import torch


def to_host(t):
    """torch tensor -> numpy array the oracle understands (float32, or uint16
    holding bfloat16 bits, or uint8 codes)."""
    if t is None:
        return None
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy()
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return t.view(torch.uint8).numpy()
    raise TypeError(t.dtype)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Float32 values -> bf16 bits via torch's cast (a library RNE)."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


def _e4m3_decode_formula(codes: np.ndarray) -> np.ndarray:
    """OCP e4m3fn decode from the format definition (sign, 4-bit exponent with
    bias 7, 3-bit mantissa; exponent 0 = subnormal; S.1111.111 = NaN)."""
    c = codes.astype(np.int64)
    s = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    v = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    v = np.where((e == 0xF) & ((c & 7) == 7), np.nan, v)
    return s * v


# value of every code, from the definition above
E4M3_TABLE = _e4m3_decode_formula(np.arange(256))
# the 127 non-negative finite values in code order, which is value order
_E4M3_POS = E4M3_TABLE[:127]


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    return E4M3_TABLE[np.asarray(codes).astype(np.intp)]


# ----------------------------------------------------------- parity rules
#
# The HIP path computes in fp32, the oracle in fp64.  The bars below bound
# the fp32 rounding of each stage and accept exactly the values that correct
# rounding of the oracle's value, perturbed within that bound, can give:
#   z (pre-norm sum): |z32 - z| <= (tp + 3) * 2^-24 * A, A = sum of |terms|
#   y (normalised):   |y32 - y| <= 2^-17 * (|y - b| + |b|) + err_z * rstd * |w|
# (2^-17 covers the fp32 sum of squares over H <= 32768 terms, the square
# root, division and the two products with margin), and then one rounding to
# the output format.  On top of this the looser published bars (bf16 within
# 1e-3 + 2^-7 |y|; per-token scales within 1e-5 relative) are asserted.

import oracle  # noqa: E402

U24 = 2.0 ** -24


def bf16_round(x: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f64(oracle.bf16_from_double_array(x))


def e4m3_round(x: np.ndarray) -> np.ndarray:
    """Nearest e4m3 value to x (float64), ties to the even mantissa, numbers
    saturated to +-448, NaN kept: a table search over the 127 non-negative
    finite values, the same rule as the oracle's brute-force encoder (checked
    equal to it on a dense sweep) at a fraction of its cost."""
    x = np.asarray(x, np.float64)
    a = np.minimum(np.abs(x), 448.0)
    i = np.clip(np.searchsorted(_E4M3_POS, a, side="left"), 1, 126)  # POS[i-1] < a <= POS[i]
    lo, hi = _E4M3_POS[i - 1], _E4M3_POS[i]
    dl, dh = a - lo, hi - a
    v = np.where((dh < dl) | ((dh == dl) & (i % 2 == 0)), hi, lo)  # code i is even: even mantissa
    return np.copysign(np.where(np.isnan(x), np.nan, v), x)


def within_rounding(got: np.ndarray, lo: np.ndarray, hi: np.ndarray, rnd) -> np.ndarray:
    """True where got lies between rnd(lo) and rnd(hi) (rounding is monotone)."""
    return (got >= rnd(lo)) & (got <= rnd(hi))


def z_error(A: np.ndarray, tp: int) -> np.ndarray:
    return (tp + 3) * U24 * A


def y_error(y, b, err_z, rstd, w):
    b = 0.0 if b is None else b
    return 2.0 ** -17 * (np.abs(y - b) + np.abs(b)) + err_z * rstd[:, None] * np.abs(w)[None, :]
