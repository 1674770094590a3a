"""Number formats used by the oracle (test infrastructure only).

* bfloat16: the upper 16 bits of an IEEE-754 binary32 value.  Decoding is a
  16-bit left shift; every bf16 value is exactly representable in fp64.
* OCP 8-bit E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits with bias 7, 3
  mantissa bits.  Exponent field 0 encodes subnormals m * 2^-9; exponent
  fields 1..15 encode (1 + m/8) * 2^(e-7), except S.1111.111 which is NaN.
  There is no infinity; the largest finite magnitude is 1.75 * 2^8 = 448.
  This is the FP8 format FlashAttention-3 computes in ("FlashAttention-3 —
  闪电注意力-3", sections on Hopper FP8 support and on low precision).
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16 / int16 array) -> fp64 values."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def e4m3_decode_table() -> np.ndarray:
    """fp64 value of each of the 256 E4M3 codes, built from the field definition."""
    out = np.empty(256, dtype=np.float64)
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            out[code] = np.nan
        elif e == 0:
            out[code] = s * m * 2.0 ** -9
        else:
            out[code] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return out


_DEC = e4m3_decode_table()
# the 127 non-negative finite codes 0x00..0x7E in increasing order of value
_POS_VALUES = _DEC[:0x7F]


def e4m3_decode(codes) -> np.ndarray:
    return _DEC[np.asarray(codes).astype(np.uint8)]


def e4m3_encode_rne(x) -> np.ndarray:
    """Round fp64 values to the nearest E4M3 code, ties to the even code.

    Magnitudes above 448 saturate to 448 (the callers scale inputs into
    [-448, 448]); NaN maps to 0x7F.  Negative values, including values that
    round to zero, carry the sign bit.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(_POS_VALUES, a, side="left")          # first code with value >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_hi = _POS_VALUES[hi] - a
    d_lo = a - _POS_VALUES[lo]
    take_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (lo % 2 == 0))
    code = np.where(take_lo, lo, hi).astype(np.uint8)
    code = np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)
    code = np.where(np.isnan(x), np.uint8(0x7F), code)
    return code
