"""IEEE binary16 helpers written out from the format definition (test infrastructure).

``value`` decodes a bit pattern to its exact value; ``round_rne`` rounds an
exact float64 value to the nearest binary16 pattern, ties to even. The code
function needs exactly these two steps: the halves produced by the mask/XOR
step are read as half-precision numbers and their sum is formed by one
half-precision add ([TQ] Part nine). Pinned against NumPy's independent
float64 -> float16 cast over every case the code function can produce.
"""
from __future__ import annotations

import numpy as np


def value(bits) -> np.ndarray:
    """Exact float64 value of binary16 bit patterns (sign, 5-bit exponent, 10-bit fraction)."""
    b = np.asarray(bits, dtype=np.int64)
    sign = np.where((b >> 15) & 1, -1.0, 1.0)
    e = (b >> 10) & 0x1F
    f = (b & 0x3FF).astype(np.float64)
    normal = np.ldexp(1024.0 + f, (e - 25).astype(np.int64))     # (1 + f/1024) * 2^(e-15)
    sub = np.ldexp(f, -24)                                         # f * 2^-24
    out = np.where(e == 0, sub, normal)
    out = np.where(e == 31, np.where(f == 0, np.inf, np.nan), out)
    return sign * out


def round_rne(v) -> np.ndarray:
    """Round float64 values to binary16 bit patterns, round-to-nearest, ties-to-even.

    Handles normals, subnormals, signed zero and overflow to infinity. NaN
    inputs are not expected by the oracle and are rejected.
    """
    v = np.asarray(v, dtype=np.float64)
    if np.isnan(v).any():
        raise ValueError("round_rne: NaN input")
    neg = np.signbit(v)
    a = np.abs(v)
    _, ex = np.frexp(np.where(a == 0, 1.0, a))           # a = mant * 2^ex, mant in [0.5, 1)
    e = np.maximum(ex - 1, -14)                           # unbiased exponent, clamped to the subnormal range
    quantum = np.ldexp(1.0, (e - 10).astype(np.int64))    # spacing of binary16 numbers at that exponent
    r = np.rint(a / quantum)                              # a / quantum is exact; rint rounds half to even
    carry = r >= 2048.0                                   # rounding overflowed the significand
    e = np.where(carry, e + 1, e)
    r = np.where(carry, r / 2, r)
    is_normal = r >= 1024.0
    field_e = np.where(is_normal, e + 15, 0)
    field_f = np.where(is_normal, r - 1024.0, r)
    bits = (field_e.astype(np.int64) << 10) | field_f.astype(np.int64)
    bits = np.where(field_e >= 31, 0x7C00, bits)          # overflow -> infinity
    bits = np.where(a == 0, 0, bits)
    bits = bits | (neg.astype(np.int64) << 15)
    return bits.astype(np.uint16)
