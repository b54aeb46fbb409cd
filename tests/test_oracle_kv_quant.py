"""Pins for the oracle's int8 K/V quantisation (CPU only).

Checked against exact rational arithmetic (fractions.Fraction) with a
hand-written binary32 rounding and Python's round-half-even, over every
finite bf16 value; plus the round-trip bound, the code range, the zero row,
and the cache-size ratio the Joy-face_change_optimized README prints.
"""
import json
import os
from fractions import Fraction

import numpy as np

from oracle import bf16_to_f64, kv_dequant, kv_quant_int8

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _round_to_binary32(fr: Fraction) -> Fraction:
    """Exact binary32 rounding (nearest, ties to even) of a rational, normal range."""
    if fr == 0:
        return Fraction(0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1                     # now 2**e <= a < 2**(e+1)
    unit = Fraction(2) ** (e - 23)  # 24 significant bits
    m = a / unit
    lo = m.numerator // m.denominator
    rem = m - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return sign * lo * unit


def _ref_row(x_vals):
    """Expected (codes, scale) of one row from exact arithmetic."""
    xs = [Fraction(float(v)) for v in x_vals]
    amax = max(abs(v) for v in xs)
    scale = _round_to_binary32(amax / 127)
    if scale == 0:
        return [0] * len(xs), scale
    codes = [max(-127, min(127, round(_round_to_binary32(v / scale)))) for v in xs]
    return codes, scale


def _all_finite_bf16_bits():
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    exp = (b >> 7) & 0xFF
    return b[(exp != 0xFF) & (exp != 0)]


def test_every_bf16_value_against_exact_arithmetic():
    bits = _all_finite_bf16_bits()
    vals = bf16_to_f64(bits)
    rng = np.random.default_rng(11)
    # rows of 128: element 0 fixes amax, the rest are every bf16 value with |x| <= amax
    for amax_bits in [0x3F80, 0x4013, 0x3B2F, 0x4420, int(rng.integers(0x3C00, 0x4400))]:
        amax = float(bf16_to_f64(np.array([amax_bits], np.uint16))[0])
        cand = bits[np.abs(vals) <= amax]
        cand = cand[rng.permutation(len(cand))]
        rows = -(-len(cand) // 127)
        cand = np.concatenate([cand, np.zeros(rows * 127 - len(cand), np.uint16)])
        x = np.concatenate([np.full((rows, 1), amax_bits, np.uint16),
                            cand.reshape(rows, 127)], axis=1)[:, None, :]
        codes, scales = kv_quant_int8(x)
        for r in range(rows):
            want_c, want_s = _ref_row(bf16_to_f64(x[r, 0]))
            assert Fraction(float(scales[r, 0])) == want_s
            assert codes[r, 0].tolist() == want_c


def test_ties_round_to_even():
    # amax = 127 gives scale exactly 1, so x/scale = x and half-integers are ties
    x = np.array([127.0, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.5, 126.5] + [0.0] * 119)
    from workloads import _f32_to_bf16_bits
    bits = _f32_to_bf16_bits(x.astype(np.float32))[None, None, :]
    codes, scales = kv_quant_int8(bits)
    assert float(scales[0, 0]) == 1.0
    assert codes[0, 0, :9].tolist() == [127, 0, 2, 2, 0, -2, -2, 4, 126]


def test_round_trip_bound_range_and_extremes():
    from workloads import normal_bf16
    x = normal_bf16(2, 3, (500, 4, 128), outlier_p=0.01, outlier_tid=9)
    codes, scales = kv_quant_int8(x)
    xv = bf16_to_f64(x)
    s = scales.astype(np.float64)[..., None]
    assert np.all(np.abs(codes.astype(np.int32)) <= 127)
    # |x - code*scale| <= scale * (1/2 + 2^-16): half a step plus the binary32
    # rounding of the quotient (|x/scale| <= 127*(1+2^-23))
    assert np.all(np.abs(xv - kv_dequant(codes, scales)) <= s * (0.5 + 2.0 ** -16))
    # the element of largest magnitude maps to +-127
    i = np.argmax(np.abs(xv), axis=-1)
    top = np.take_along_axis(codes, i[..., None], -1)[..., 0]
    assert np.all(np.abs(top.astype(np.int32)) == 127)
    # scale is the binary32 quotient amax / 127
    amax = np.abs(xv).max(-1)
    assert np.array_equal(scales, np.float32(amax / 127.0))


def test_zero_row():
    x = np.zeros((2, 3, 64), np.uint16)
    x[1, 2, 5] = 0x3F80
    codes, scales = kv_quant_int8(x)
    assert scales[0].tolist() == [0.0, 0.0, 0.0] and scales[1, :2].tolist() == [0.0, 0.0]
    assert not codes[0].any() and codes[1, 2, 5] == 127


def test_cache_size_ratio_matches_the_page():
    g = json.load(open(os.path.join(GOLDEN, "kv_cache_size.json")))
    d = g["head_dim"]
    codes, scales = kv_quant_int8(np.zeros((1, 1, d), np.uint16))
    per_row_int8 = codes.itemsize * d + scales.itemsize
    per_row_bf16 = 2 * d
    got = round(g["bf16_cache_gib"] * per_row_int8 / per_row_bf16, g["printed_decimals"])
    assert got == g["int8_cache_gib"]
    # a 2-byte scale would not reproduce the printed figure
    assert round(g["bf16_cache_gib"] * (d + 2) / per_row_bf16, 2) != g["int8_cache_gib"]
