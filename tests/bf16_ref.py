"""Exact, independent bf16 rounding for tests (rational arithmetic).

Used only to check the oracle's bf16 rounding and by brute-force tests; it
works on Python Fractions, so it shares no arithmetic with the C oracle."""
from fractions import Fraction
import math


def bf16_bits_of_fraction(v: Fraction) -> int:
    """Round an exact rational to bf16, nearest with ties to even."""
    if v == 0:
        return 0
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    # exponent e with 2^e <= a < 2^(e+1)
    e = math.floor(math.log2(a.numerator)) - math.floor(math.log2(a.denominator))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    q = max(e - 7, -133)                    # weight of the last kept bit
    scaled = a / (Fraction(2) ** q)
    fl = scaled.numerator // scaled.denominator
    rem = scaled - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    val = Fraction(fl) * Fraction(2) ** q
    if val >= Fraction(2) ** 128:
        return sign | 0x7F80
    if val < Fraction(2) ** -126:           # subnormal: mantissa = val / 2^-133
        return sign | int(val / Fraction(2) ** -133)
    ev = math.floor(math.log2(val.numerator)) - math.floor(math.log2(val.denominator))
    while Fraction(2) ** ev > val:
        ev -= 1
    while Fraction(2) ** (ev + 1) <= val:
        ev += 1
    mant = int(val / Fraction(2) ** (ev - 7)) - 128
    return sign | ((ev + 127) << 7) | mant


def bf16_value(bits: int) -> float:
    """Decode a bf16 bit pattern to a Python float (exact)."""
    import struct
    return struct.unpack("<f", struct.pack("<I", (bits & 0xFFFF) << 16))[0]
