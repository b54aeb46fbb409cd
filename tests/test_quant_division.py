"""The int8 quantiser's quotient x / scale without a division per element.

For every row scale the kernel can meet on its fast path (scale =
fl32(amax / 127) with amax a bf16 value, scale >= 2^-100) and every bf16 x
with |x| <= amax, the kernel's sequence
    y  = RN32(1 / scale)
    q0 = RN32(x * y)
    r  = RN32(x - q0 * scale)      one fma
    q  = RN32(q0 + r * y)          one fma
must give the defined codes clamp(rint(RN32(x / scale)), -127, 127).
Where |x / scale| >= 1/8 every intermediate is normal (x >= scale/8 >=
2^-103, the residual is about ulp(q) * scale >= 2^-126), and Markstein's
theorem gives q = RN32(x / scale) exactly: checked bit for bit there. Below
1/8 the residual may underflow and q may be off by some ulps, but it stays
far below the first rounding boundary 1/2, so the code is 0 either way:
checked on the codes. Exact arithmetic, every positive bf16 x against about
2000 scales; the sequence is odd in x, so negative x follow. Host arithmetic
only: the GPU tests check the kernel's codes bit for bit against the oracle."""
from fractions import Fraction

import numpy as np


def _bf16(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32)


def _rn32_exact(v: Fraction) -> np.float32:
    """Round an exact rational to binary32, nearest, ties to even (normal range)."""
    if v == 0:
        return np.float32(0.0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    m = a / Fraction(2) ** (e - 23)            # in [2^23, 2^24)
    n, rem = divmod(m.numerator, m.denominator)
    twice = 2 * rem
    if twice > m.denominator or (twice == m.denominator and n % 2 == 1):
        n += 1
    return np.float32(sign * float(Fraction(n) * Fraction(2) ** (e - 23)))


def _kernel_quotient(x: np.ndarray, scale: np.float32) -> np.ndarray:
    y = np.float32(1.0 / np.float64(scale))               # RN32(1/scale): no binary32 tie is reachable
    q0 = (x * y).astype(np.float32)                        # binary32 product
    r = (x.astype(np.float64) - q0.astype(np.float64) * np.float64(scale)).astype(np.float32)  # exact, then RN32
    s = q0.astype(np.float64) + r.astype(np.float64) * np.float64(y)  # r*y exact; the sum may round once in fp64
    q = s.astype(np.float32)
    # the fp64 sum's rounding can only change RN32 when it lands on (or next to)
    # a binary32 half-way point: redo those few exactly
    low = s.view(np.uint64) & np.uint64((1 << 29) - 1)
    near = np.abs(low.astype(np.int64) - (1 << 28)) <= 2
    for i in np.nonzero(near)[0]:
        exact = Fraction(float(q0[i])) + Fraction(float(r[i])) * Fraction(float(y))
        q[i] = _rn32_exact(exact)
    return q


def test_rn32_exact_rounding_helper():
    one = Fraction(1)
    ulp = Fraction(1, 2 ** 23)
    assert _rn32_exact(one + ulp / 2) == np.float32(1.0)             # tie to even (down)
    assert _rn32_exact(one + ulp + ulp / 2) == np.float32(1.0) + np.float32(2.0 ** -22)   # tie to even (up)
    assert _rn32_exact(one + ulp / 2 + Fraction(1, 2 ** 40)) == np.float32(1.0) + np.float32(2.0 ** -23)
    assert _rn32_exact(Fraction(-3, 7)) == np.float32(-3.0) / np.float32(7.0)


def test_quotient_without_division_is_correctly_rounded():
    pos = np.arange(1, 0x7F80, dtype=np.uint32)                     # every positive finite bf16
    xs_all = _bf16(pos)
    # scales: a stride through every bf16 amax, plus all-ones and all-zeros
    # mantissas at every exponent (the extreme reciprocals)
    amax_bits = set(range(1, 0x7F80, 17))
    for e in range(1, 255):
        amax_bits |= {(e << 7) | 0x7F, (e << 7), (e << 7) | 0x01, (e << 7) | 0x40}
    checked = 0
    for ab in sorted(amax_bits):
        amax = _bf16([ab])[0]
        scale = np.float32(amax) / np.float32(127.0)
        if not scale >= np.float32(2.0 ** -100):
            continue                                                 # those rows divide per element
        xs = xs_all[xs_all <= amax]
        want = xs / scale                                            # IEEE binary32 division
        got = _kernel_quotient(xs, scale)
        exact = want >= np.float32(0.125)
        bad = np.nonzero(exact & (got.view(np.uint32) != want.view(np.uint32)))[0]
        assert bad.size == 0, (float(amax), float(xs[bad[0]]), float(got[bad[0]]), float(want[bad[0]]))
        code_got = np.clip(np.rint(got), -127, 127)
        code_want = np.clip(np.rint(want), -127, 127)
        assert np.array_equal(code_got, code_want), float(amax)
        assert np.all(got[~exact] < np.float32(0.25))
        checked += xs.size
    assert checked > 20_000_000
