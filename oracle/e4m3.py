"""OCP OFP8 E4M3 codec (torch's ``float8_e4m3fn``), from the format definition.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The PR 31340 digest ("Fix FP8 Triton dtype selection on A100", section "Key
source excerpts", ``fp8_dtype_to_triton``) names the activation/weight format as
``float8_e4m3fn``: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, no
infinities, NaN only at S.1111.111, largest finite magnitude 448.

The PR 27896 digest ("Key source excerpts", the row-padded quant function)
hands ``fp8_min`` / ``fp8_max`` to the quantization kernel, i.e. values are
clamped into the finite range before conversion; the pages do not state the
rounding mode, and the reading taken is IEEE round-to-nearest, ties to the even
significand.
"""

import numpy as np

E4M3_MAX = 448.0


def _value_of(code: int) -> float:
    """Exact value of one 8-bit E4M3 code (float64; NaN for the two NaN codes)."""
    sign = -1.0 if code & 0x80 else 1.0
    exponent = (code >> 3) & 0xF
    mantissa = code & 0x7
    if exponent == 0xF and mantissa == 0x7:
        return float("nan")
    if exponent == 0:  # subnormal: 0.mmm * 2^(1-7)
        return sign * (mantissa / 8.0) * 2.0 ** -6
    return sign * (1.0 + mantissa / 8.0) * 2.0 ** (exponent - 7)


def decode_table() -> np.ndarray:
    """float64[256]: the value of every code (NaN at 0x7F and 0xFF)."""
    return np.array([_value_of(c) for c in range(256)], dtype=np.float64)


_TABLE = decode_table()
# The 127 non-negative finite values, codes 0x00..0x7E, ascending.
_POS = _TABLE[:0x7F].copy()


def decode(codes) -> np.ndarray:
    """Decode an array of uint8 codes to float64."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def encode(v) -> np.ndarray:
    """fp32 values -> uint8 E4M3 codes.

    Saturating: the value is first clamped to [-448, 448]; it is then rounded to
    the nearest representable magnitude, a tie going to the code whose
    significand is even (its lowest bit is 0). The sign bit is copied from the
    input, so -0.0 and negative values that round to zero give 0x80.
    Non-finite inputs are outside the method (parity unpinned).
    """
    v32 = np.asarray(v, dtype=np.float32)
    mag = np.abs(v32.astype(np.float64))
    mag = np.minimum(mag, E4M3_MAX)
    neg = np.signbit(v32)

    # hi = first code whose value is >= mag; lo = the one below it.
    hi = np.searchsorted(_POS, mag, side="left")
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = mag - _POS[lo]
    d_hi = _POS[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((hi & 1) == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    # exact hits (including 0) land on hi with d_hi == 0 <= d_lo
    return (code | (neg.astype(np.uint8) << 7)).astype(np.uint8)
