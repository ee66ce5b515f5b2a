"""FP8 E4M3 ("e4m3fn") codec, from the OCP 8-bit floating point format definition.

The pages only say the cache is FP8 with per-head scales (cpdf.ai blog, sections "Como
rodar 57B..." and "Blackwell, escalabilidade..."); the exact format is a reading: the OCP
E4M3 variant, which gfx950 converts to natively.

Format: bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0 mantissa.  Exponent field 0
encodes subnormals m * 2^-9; otherwise (1 + m/8) * 2^(e-7).  There are no infinities; the
codes 0x7F and 0xFF are NaN, so the largest finite magnitude is 448 (0x7E).

Encoding rule (reading): round to the nearest representable value, ties to the code with
the even mantissa; magnitudes above 448 saturate to 448; the sign of the input (including
the sign of zero) is kept.  Inputs are finite.
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode_table() -> np.ndarray:
    """float64 value of each of the 256 codes, straight from the field definitions."""
    t = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            t[code] = np.nan
        elif e == 0:
            t[code] = sign * m * 2.0 ** -9
        else:
            t[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return t


_TABLE = e4m3_decode_table()
# The 127 non-negative finite values, codes 0x00..0x7E, strictly increasing with the code.
_POS_VALUES = _TABLE[:0x7F].copy()
assert np.all(np.diff(_POS_VALUES) > 0)


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """uint8 codes -> float64 values (exact)."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """float32 (or float64 holding float32 values) -> uint8 codes.

    Nearest-value search over the 127 non-negative finite values; an exact tie goes to the
    even code (codes of consecutive magnitudes are consecutive, so the even code is the even
    mantissa); |x| > 448 saturates; the sign bit of x is copied."""
    x = np.asarray(x)
    a = np.minimum(np.abs(x.astype(np.float64)), E4M3_MAX)
    hi = np.searchsorted(_POS_VALUES, a, side="left")       # first value >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((hi & 1) == 0))
    code = np.where(take_hi, hi, lo).astype(np.uint8)
    sign = np.signbit(x).astype(np.uint8) << np.uint8(7)
    return (code | sign).astype(np.uint8)
