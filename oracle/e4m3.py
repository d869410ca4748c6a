"""OCP FP8 E4M3 ("fn") codec -- test infrastructure only (see ``oracle/__init__``).

Reading of the pages: "FP8 ViT Encoder Attention" (intro) and "FP8 vision
encoder attention" (Requirements) say only "FP8" and name a path for MI300 and
MI350 (gfx942 and gfx950).  The format taken here is OCP E4M3 "fn", the one
gfx950's conversion instructions produce:

* 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
* exponent field 0 encodes subnormals ``m * 2**-9``;
* no infinities; ``S.1111.111`` (0x7F, 0xFF) is NaN;
* largest finite magnitude ``S.1111.110`` = 448.

Encoding rounds to nearest, ties to even, saturates to +-448 (Inf included),
and keeps the sign of zero.  NaN inputs are rejected.
"""

import numpy as np

FP8_MAX = 448.0


def _decode_code(code: int) -> float:
    """Value of one 8-bit code, straight from the field definitions."""
    sign = -1.0 if code & 0x80 else 1.0
    exp_field = (code >> 3) & 0xF
    mant = code & 0x7
    if exp_field == 0xF and mant == 0x7:
        return float("nan")
    if exp_field == 0:
        return sign * mant * 2.0 ** -9          # subnormal: (m/8) * 2**(1-7)
    return sign * (1.0 + mant / 8.0) * 2.0 ** (exp_field - 7)


#: float64 value of every code 0..255 (NaN at 0x7F and 0xFF).
DECODE_TABLE = np.array([_decode_code(c) for c in range(256)], dtype=np.float64)

# Codes 0x00..0x7E are the non-negative finite values in increasing order.
_POSITIVE = DECODE_TABLE[:0x7F]


def decode(codes) -> np.ndarray:
    """Codes (any integer array) -> float64 values."""
    c = np.asarray(codes)
    return DECODE_TABLE[c.astype(np.uint8)]


def encode(y) -> np.ndarray:
    """float32 array -> uint8 E4M3 codes (RNE, saturating, signed zero).

    Steps: ``a = min(|y|, 448)``; the spacing of representable values around
    ``a`` is ``2**-9`` below the smallest normal ``2**-6`` and
    ``2**(floor(log2 a) - 3)`` above it; round ``a`` to a multiple of that
    spacing with ties to even; look the result up among the non-negative
    codes; set the sign bit from ``y``.  Clamping before rounding gives the
    same result as rounding then saturating, because 448 is itself
    representable and the next value up would be 480.
    """
    y = np.asarray(y, dtype=np.float32)
    if np.isnan(y).any():
        raise ValueError("NaN has no saturating E4M3 encoding here")
    a = np.minimum(np.abs(y.astype(np.float64)), FP8_MAX)
    _, e = np.frexp(a)                       # a = f * 2**e, f in [0.5, 1)
    spacing = np.where(a < 2.0 ** -6, 2.0 ** -9, np.ldexp(1.0, e - 4))
    v = np.rint(a / spacing) * spacing       # np.rint rounds half to even
    idx = np.searchsorted(_POSITIVE, v)
    idx = np.minimum(idx, len(_POSITIVE) - 1)
    if not np.array_equal(_POSITIVE[idx], v):
        raise AssertionError("rounded value is not an E4M3 value")
    sign = np.where(np.signbit(y), 0x80, 0x00)
    return (idx | sign).astype(np.uint8)
