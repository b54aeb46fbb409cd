"""The fp64 sin/cos of the rotary kernel reduces its argument by pi/2 split
into three doubles (Cody and Waite). The constants in
streaming_video_dit_amd/csrc/qknorm_rope3d.hip are checked here against pi
computed from Machin's formula in exact integer arithmetic: the first two
parts have at most 33 significant bits (so k times them is exact for
|k| < 2^20), the three add up to pi/2 within 2^-115, and 2/pi is the double
nearest to it."""
import math
import os
import re
from fractions import Fraction

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "streaming_video_dit_amd", "csrc", "qknorm_rope3d.hip")


def _pi(digits=90):
    def arctan_inv(x):
        scale = 10 ** digits
        total = term = scale // x
        n, sign = 1, -1
        while term:
            term //= x * x
            total += sign * (term // (2 * n + 1))
            sign, n = -sign, n + 1
        return total
    return Fraction(4 * (4 * arctan_inv(5) - arctan_inv(239)), 10 ** digits)


def _constant(name):
    m = re.search(r"constexpr double %s = (0x[0-9a-fA-F.]+p[-+]?\d+);" % name, open(SRC).read())
    assert m, name
    return float.fromhex(m.group(1))


def _significant_bits(x):
    m, _ = math.frexp(x)
    f = Fraction(m)
    return f.denominator.bit_length() - 1


def test_pi_from_machin_is_right():
    assert abs(float(_pi()) - math.pi) == 0.0


def test_pi_over_2_split():
    half_pi = _pi() / 2
    a, b, c = (_constant(n) for n in ("kPio2a", "kPio2b", "kPio2c"))
    assert _significant_bits(a) <= 33 and _significant_bits(b) <= 33
    assert abs(half_pi - (Fraction(a) + Fraction(b) + Fraction(c))) < Fraction(1, 2 ** 115)
    # each part is the best value of its kind: a and b rounded to 33 bits, c to nearest double
    assert abs(half_pi - Fraction(a)) <= Fraction(1, 2 ** 33)
    assert Fraction(c) == Fraction(float(half_pi - Fraction(a) - Fraction(b)))


def test_two_over_pi_is_correctly_rounded():
    t = _constant("kTwoOverPi")
    exact = 2 / _pi()
    ulp = math.ulp(t)
    assert abs(Fraction(t) - exact) <= Fraction(ulp) / 2
