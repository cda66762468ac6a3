"""FP8 E4M3 codec of the projected-key cache, written from the format definition.

Test infrastructure only (see the package docstring).

The JSSA article (section "How JSSA preserves token order") keeps the
projected-key cache in FP8 but does not name the flavour.  Reading taken: the
OCP 8-bit floating point E4M3 format ("e4m3fn"): 1 sign bit, 4 exponent bits
with bias 7, 3 mantissa bits, no infinities, NaN only for the two codes with
all exponent and mantissa bits set (0x7F, 0xFF), largest finite magnitude 448.

Encoding rounds to nearest with ties to the even mantissa and saturates
magnitudes above 448 to +-448 ("satfinite").  NaN input is an error.
"""

import numpy as np

FP8_MAX = 448.0
_EXP_BIAS = 7
_MANT_BITS = 3
_MIN_NORMAL_EXP = 1 - _EXP_BIAS          # 2**-6 is the smallest normal
_SUBNORMAL_STEP = 2.0 ** (_MIN_NORMAL_EXP - _MANT_BITS)   # 2**-9


def _decode_code(c: int) -> float:
    """Value of one code, straight from the field definition."""
    sign = -1.0 if (c >> 7) & 1 else 1.0
    e = (c >> _MANT_BITS) & 0xF
    m = c & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** _MIN_NORMAL_EXP
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - _EXP_BIAS)


_TABLE = np.array([_decode_code(c) for c in range(256)], dtype=np.float64)


def decode_table() -> np.ndarray:
    """All 256 code values (float64, index = code byte)."""
    return _TABLE.copy()


def fp8_decode(codes) -> np.ndarray:
    """uint8 codes -> float64 values (exact)."""
    codes = np.asarray(codes, dtype=np.uint8)
    return _TABLE[codes]


def fp8_encode(x) -> np.ndarray:
    """float64 values -> uint8 codes, round-to-nearest-even, saturating.

    The sign of the code is the sign bit of the input, so -0.0 encodes as 0x80.
    """
    x = np.asarray(x, dtype=np.float64)
    if np.isnan(x).any():
        raise ValueError("fp8_encode: NaN input")
    sign = np.signbit(x).astype(np.uint8) << 7
    a = np.abs(x)
    code = np.zeros(a.shape, dtype=np.int64)

    sat = a >= FP8_MAX
    sub = a < 2.0 ** _MIN_NORMAL_EXP
    nrm = ~(sat | sub)

    # Subnormal range: value = m * 2**-9, m in 0..7; rounding may reach m = 8,
    # whose bit pattern 0b0001000 is exactly the smallest normal (2**-6).
    code[sub] = np.rint(a[sub] / _SUBNORMAL_STEP).astype(np.int64)

    # Normal range: a = f * 2**e with f in [1, 2).  All steps are exact in
    # float64 (power-of-two scaling, subtracting 1, multiplying by 8).
    mant, exp2 = np.frexp(a[nrm])          # a = mant * 2**exp2, mant in [0.5, 1)
    e = exp2.astype(np.int64) - 1
    q = np.rint((2.0 * mant - 1.0) * 8.0).astype(np.int64)
    carry = q == 8
    e = np.where(carry, e + 1, e)
    q = np.where(carry, 0, q)
    biased = e + _EXP_BIAS
    over = (biased > 15) | ((biased == 15) & (q == 7))
    c_nrm = (biased << _MANT_BITS) | q
    c_nrm = np.where(over, 0x7E, c_nrm)
    code[nrm] = c_nrm

    code[sat] = 0x7E
    return (code.astype(np.uint8) | sign).astype(np.uint8)
