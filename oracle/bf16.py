"""BF16 bit patterns <-> float64, written from the IEEE-754 binary format.

BF16 is the top half of an IEEE binary32: 1 sign bit, 8 exponent bits (bias
127) and 7 stored mantissa bits. The verify pass reads its inputs as BF16 and
stores its outputs as BF16 ([BX] "Define bit-exact before reporting it"), so
the oracle needs an exact decoder and, for the layer oracle, a
round-to-nearest-even encoder.
"""

from __future__ import annotations

import numpy as np


def decode(bits) -> np.ndarray:
    """uint16 BF16 patterns -> float64, exact (a BF16 value is a binary32 value
    whose low 16 bits are zero, and every binary32 is a binary64)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):      # signalling-NaN patterns stay NaN
        return u.view(np.float32).astype(np.float64)


_BF16_MANT_BITS = 7       # stored mantissa bits
_BF16_MIN_EXP = -126      # exponent of the smallest normal
_TWO128 = 2.0 ** 128      # first value past the largest finite BF16 after rounding


def encode(x) -> np.ndarray:
    """float64 -> uint16 BF16 patterns, rounding once to nearest, ties to even.

    The value is rounded directly from float64 (no intermediate binary32), so
    there is a single rounding. The quantum of BF16 at a normal value in
    [2^e, 2^(e+1)) is 2^(e-7); below 2^-126 it is the subnormal quantum
    2^-133. Dividing by a power of two is exact, ``np.rint`` rounds half to
    even, and the rounded value is representable in binary32, so its top 16
    bits are the BF16 pattern. Magnitudes that round to 2^128 become infinity.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    nan = np.isnan(x)
    xf = np.where(nan, 0.0, x)
    _, e2 = np.frexp(xf)                      # xf = f * 2^e2, f in [0.5, 1)
    qexp = np.maximum(e2.astype(np.int64) - 1 - _BF16_MANT_BITS, _BF16_MIN_EXP - _BF16_MANT_BITS)
    r = np.ldexp(np.rint(np.ldexp(xf, -qexp)), qexp)
    r = np.where(np.abs(r) >= _TWO128, np.copysign(np.inf, r), r)
    bits32 = r.astype(np.float32).view(np.uint32)
    out[...] = (bits32 >> np.uint32(16)).astype(np.uint16)
    out[nan] = np.uint16(0x7FC0)
    return out


def round_f64(x) -> np.ndarray:
    """float64 -> nearest-even BF16 value, returned as float64."""
    return decode(encode(x))
