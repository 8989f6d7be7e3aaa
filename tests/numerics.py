"""Exact-rounding and ulp helpers shared by the tests.

They are test utilities, independent of both the oracle and the HIP library:
each is written from the definition of IEEE rounding, and
tests/test_oracle_pins.py pins each one to torch's own conversions.
"""
from fractions import Fraction

import numpy as np


def bf16_bits_to_f32(b) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float32 values (exact widening)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f64_to_bf16_exact(v) -> np.ndarray:
    """Round float64 values directly to bfloat16 (nearest, ties to even), with no
    intermediate float32 rounding. Returns uint16 bit patterns; NaN -> 0x7FC0
    with the input's sign."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    finite = np.isfinite(a)
    a_f = np.where(finite, a, 0.0)
    _, e = np.frexp(a_f)                      # a = m * 2**e, m in [0.5, 1)
    lead = e - 1                              # exponent of the leading bit
    q = np.maximum(lead, -126) - 7            # exponent of one bfloat16 ulp
    r = np.rint(np.ldexp(a_f, -q))            # ties to even
    val = np.ldexp(r, q)
    with np.errstate(over="ignore"):
        f32 = val.astype(np.float32)          # exact, or inf when val >= 2**128
    f32 = np.where(finite, f32, np.float32(np.inf)).astype(np.float32)
    f32 = np.copysign(f32, v).astype(np.float32)
    bits = (f32.view(np.uint32) >> 16).astype(np.uint16)
    nan = np.isnan(v)
    bits = np.where(nan, np.where(np.signbit(v), 0xFFC0, 0x7FC0), bits).astype(np.uint16)
    return bits


def fraction_to_f32(q: Fraction) -> np.float32:
    """Round an exact rational to float32 (nearest, ties to even)."""
    if q == 0:
        return np.float32(0.0)
    neg = q < 0
    a = -q if neg else q
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    qe = max(e, -126) - 23
    scaled = a / (Fraction(2) ** qe)
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    val = Fraction(n) * Fraction(2) ** qe
    if val >= Fraction(2) ** 128:
        out = np.float32(np.inf)
    else:
        out = np.float32(float(val))          # exact: n has at most 24 bits
    return np.float32(-out) if neg else out


def bf16_order(b) -> np.ndarray:
    """Map bfloat16 bit patterns to integers that are ordered like the values
    (+0 and -0 both map to 0), so |order(a) - order(b)| is the ulp distance."""
    b = np.asarray(b, dtype=np.uint16).astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def bf16_ulp_diff(a, b) -> np.ndarray:
    return np.abs(bf16_order(a) - bf16_order(b))


def bf16_is_nan(b) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint16)
    return ((b & 0x7F80) == 0x7F80) & ((b & 0x007F) != 0)


def f16_is_nan(b) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint16)
    return ((b & 0x7C00) == 0x7C00) & ((b & 0x03FF) != 0)


def f32_ulp(x) -> np.ndarray:
    """Size of one float32 ulp at |x|."""
    x = np.abs(np.asarray(x, dtype=np.float32))
    return (np.nextafter(x, np.float32(np.inf), dtype=np.float32) - x).astype(np.float64)
