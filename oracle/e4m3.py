"""OCP FP8 E4M3FN codes (test infrastructure only; see oracle/__init__).

The pages ask for an FP8 path ([FA3-V3] §4.3; [FA3-card] "低精度优化") but do
not define the format, and the simulation printed in [FA3-V3] §11
(``fp32_to_fp8_conversion``: clamp to ±240, round to a 1/16 grid) is not an
FP8 format at all.  The reading taken is the OCP 8-bit E4M3FN encoding, the one
gfx950's matrix cores consume:

* bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0 mantissa;
* exponent 0: subnormal, value = m/8 · 2^-6 (smallest 2^-9);
* exponent 1..15: value = (1 + m/8) · 2^(e-7); S.1111.111 is NaN, so the
  largest finite magnitude is 1.75 · 2^8 = 448; there is no infinity.

Conversion: round to nearest, ties to even mantissa, saturating to ±448 (never
NaN for finite input); the sign of a value that rounds to zero is kept (0x80).
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def decode_table() -> np.ndarray:
    """The 256 code values as fp64 (NaN for 0x7F and 0xFF)."""
    vals = np.empty(256)
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            vals[c] = np.nan
        elif e == 0:
            vals[c] = s * (m / 8.0) * 2.0 ** -6
        else:
            vals[c] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_TABLE = decode_table()
_POS = _TABLE[:0x7F]          # codes 0x00..0x7E: 0 .. 448, strictly increasing


def decode(codes) -> np.ndarray:
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def encode(x) -> np.ndarray:
    """Round fp values (any float dtype, finite) to E4M3FN codes, RNE, saturating."""
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("encode() takes finite values only")
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(_POS, a, side="left")        # first code with value >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    dlo = a - _POS[lo]
    dhi = _POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a == _POS[hi], hi, code)           # exact hits
    sign = np.signbit(x).astype(np.int64) << 7
    return (code | sign).astype(np.uint8)
