"""Exact decoding of the storage formats to float64 (oracle; test infrastructure).

The decode is written from the formats' bit-level definitions, not from any
library conversion, so that it can be checked against torch's casts as an
independent pin.

* bfloat16: the upper 16 bits of an IEEE-754 binary32 value.  Widening to
  binary32 by appending 16 zero bits is exact, and binary32 -> float64 is
  exact.
* fp8 E4M3FN (OCP "FN" variant, the one the long-context fp8 workload of the
  pages' FP8-KV path uses): 1 sign bit, 4 exponent bits with bias 7, 3
  mantissa bits; exponent field 0 encodes subnormals (m/8 * 2^-6); the all-ones
  exponent with all-ones mantissa (S.1111.111) is NaN; there is no infinity, so
  S.1111.000 .. S.1111.110 are ordinary normals up to 448.
"""

import numpy as np


def bf16_bits_to_f64(bits):
    """uint16 bf16 codes -> float64 (exact)."""
    b = np.asarray(bits)
    if b.dtype != np.uint16:
        b = b.astype(np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _e4m3fn_value(code):
    sign = -1.0 if (code >> 7) & 1 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        return sign * (man / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


def e4m3fn_table():
    """float64[256]: value of each E4M3FN code, NaN for the two NaN codes."""
    return np.array([_e4m3fn_value(c) for c in range(256)], dtype=np.float64)


_E4M3FN = e4m3fn_table()


def e4m3fn_bits_to_f64(bits):
    """uint8 E4M3FN codes -> float64 (exact, table lookup)."""
    b = np.asarray(bits)
    if b.dtype != np.uint8:
        b = b.astype(np.uint8)
    return _E4M3FN[b]
