"""Exact-rational restatement of the INT8 row quantizer, used to pin the oracle.

It does not use floating-point division at all: every value is a Fraction,
and rounding to IEEE binary32 (nearest, ties to even, with subnormals) is
done by integer arithmetic.  Definition being pinned: scale = fp32(amax/127),
q = round_half_even(fp32(x/scale)) clamped to [-127, 127]; zero row -> 0.
"""
from fractions import Fraction


def bf16_to_fraction(bits: int) -> Fraction:
    bits &= 0xFFFF
    sign = -1 if bits & 0x8000 else 1
    e = (bits >> 7) & 0xFF
    m = bits & 0x7F
    if e == 0xFF:
        raise ValueError("non-finite")
    if e == 0:
        v = Fraction(m, 1 << 7) * Fraction(1, 1 << 126)
    else:
        v = Fraction(128 + m, 128) * (Fraction(2) ** (e - 127))
    return sign * v


def _round_half_even(r: Fraction) -> int:
    fl = r.numerator // r.denominator
    rem = r - fl
    if rem > Fraction(1, 2):
        return fl + 1
    if rem < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


def round_to_f32(r: Fraction) -> Fraction:
    """Nearest binary32 value to r (ties to even), subnormals kept, no overflow handling."""
    if r == 0:
        return Fraction(0)
    sign = -1 if r < 0 else 1
    a = abs(r)
    # exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    if Fraction(2) ** (e + 1) <= a:
        e += 1
    quantum_exp = max(e, -126) - 23  # ulp exponent; subnormal ulp is 2^-149
    quantum = Fraction(2) ** quantum_exp
    n = _round_half_even(a / quantum)
    return sign * n * quantum


def f32_bits(v: Fraction) -> int:
    import struct
    return struct.unpack("<I", struct.pack("<f", float(v)))[0]


def quantize_row_exact(bits_row):
    """Returns (list of int q, Fraction scale)."""
    xs = [bf16_to_fraction(b) for b in bits_row]
    amax = max(abs(x) for x in xs)
    if amax == 0:
        return [0] * len(xs), Fraction(0)
    scale = round_to_f32(amax / 127)
    q = []
    for x in xs:
        y = round_to_f32(x / scale)
        qi = _round_half_even(y)
        q.append(max(-127, min(127, qi)))
    return q, scale
