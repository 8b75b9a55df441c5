"""OCP FP8 E4M3 codec in plain NumPy (test infrastructure; see package header).

The pages only say that the KV cache may be stored in FP8 ([vLLM-history] §5.2,
§7.3). The format taken is E4M3 as defined by the OCP "8-bit Floating Point
Specification (OFP8)" v1.0:

* 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits;
* exponent field 0 holds subnormals m · 2^-9 (m = 0..7), so the smallest
  positive value is 2^-9 and the smallest normal is 2^-6;
* exponent field 15 with mantissa 111 is NaN (both signs); there is no
  infinity, so S.1111.110 = ±448 is the largest finite value.

Encoding reading (the pages fix none of it): round to nearest, ties to even, on
the E4M3 grid; magnitudes above 448 (including infinity) saturate to ±448; NaN
stays NaN (code 0x7F, or 0xFF when the sign bit is set); the sign bit of the
input is kept, so a negative value that rounds to zero becomes code 0x80.
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
_MIN_NORMAL = 2.0 ** -6
_SUBNORMAL_QUANTUM = 2.0 ** -9


def e4m3_code_values() -> np.ndarray:
    """Value of every code 0..255 as float64 (NaN for S.1111.111).

    Built field by field from the format definition: sign, exponent with bias
    7, three mantissa bits, subnormals at exponent field 0.
    """
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        exp_field = (code >> 3) & 0xF
        mant = code & 0x7
        if exp_field == 0xF and mant == 0x7:
            vals[code] = np.nan
        elif exp_field == 0:
            vals[code] = sign * mant * _SUBNORMAL_QUANTUM
        else:
            vals[code] = sign * (1.0 + mant / 8.0) * 2.0 ** (exp_field - 7)
    return vals


_VALUES = e4m3_code_values()
# Positive finite magnitudes in code order 0x00..0x7E; they increase strictly,
# so a magnitude that lies on the grid is found by binary search.
_POS_MAGNITUDES = _VALUES[:0x7F].copy()


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Exact float64 value of each uint8 code."""
    codes = np.asarray(codes)
    if codes.dtype != np.uint8:
        raise TypeError("e4m3_decode expects uint8 codes")
    return _VALUES[codes]


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Encode float32 values to E4M3 codes (RNE, saturating, sign kept).

    Every step is exact in float64: a float32 magnitude divided by a power of
    two is exact, and ``np.rint`` rounds halves to even.
    """
    x = np.asarray(x)
    if x.dtype != np.float32:
        raise TypeError("e4m3_encode expects float32 input")
    a = np.abs(x.astype(np.float64))
    nan = np.isnan(a)
    a = np.where(nan, 0.0, a)
    # Spacing of the E4M3 grid around a: 2^(e-3) for a normal value in
    # [2^e, 2^(e+1)), and 2^-9 across the whole subnormal range.
    _, e_plus_1 = np.frexp(np.maximum(a, _MIN_NORMAL))
    quantum = np.ldexp(1.0, e_plus_1 - 1 - 3)
    quantum = np.where(a < _MIN_NORMAL, _SUBNORMAL_QUANTUM, quantum)
    with np.errstate(invalid="ignore"):
        mag = np.rint(a / quantum) * quantum
    mag = np.where(a > E4M3_MAX, E4M3_MAX, mag)  # saturation (also catches inf)
    mag = np.minimum(mag, E4M3_MAX)
    code = np.searchsorted(_POS_MAGNITUDES, mag).astype(np.uint8)
    if not np.array_equal(_POS_MAGNITUDES[code], mag):
        raise AssertionError("E4M3 rounding left the grid")  # cannot happen
    code = np.where(nan, np.uint8(0x7F), code).astype(np.uint8)
    sign = np.signbit(x).astype(np.uint8) << 7
    return (code | sign).astype(np.uint8)
