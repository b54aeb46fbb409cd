"""Pins for the oracle's bf16 conversions (CPU only).

bf16 is the top half of a binary32 word; rounding from fp64 is to nearest,
ties to even. Checked against brute force over the full table of bf16
values, independent of the oracle's frexp-based rounding.
"""
import numpy as np
import pytest

from oracle import bf16_to_f64, f64_to_bf16


def _finite_table():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    exp = (bits >> 7) & 0xFF
    ok = (exp != 0xFF) & ((exp != 0) | ((bits & 0x7F) == 0))  # finite, no subnormals
    bits = bits[ok]
    vals = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return bits, vals


def test_widen_is_binary32_upper_half():
    bits, vals = _finite_table()
    # 1.0 = 0x3F80, -2.0 = 0xC000, 0.5 = 0x3F00 (binary32 layout)
    assert bf16_to_f64(np.array([0x3F80, 0xC000, 0x3F00], np.uint16)).tolist() == [1.0, -2.0, 0.5]
    assert np.array_equal(bf16_to_f64(bits), vals)


def test_round_trip_every_finite_bf16():
    bits, vals = _finite_table()
    back = f64_to_bf16(vals)
    # +0 and -0 both come back as a zero; compare values, and bits off zero
    nz = vals != 0
    assert np.array_equal(back[nz], bits[nz])
    assert np.all(bf16_to_f64(back[~nz]) == 0)


def test_rounding_matches_brute_force_nearest_even():
    bits, vals = _finite_table()
    order = np.argsort(vals, kind="stable")
    sv, sb = vals[order], bits[order]
    # drop -0 duplicate of +0 for the search table
    keep = np.concatenate([[True], sv[1:] != sv[:-1]])
    sv, sb = sv[keep], sb[keep]
    rng = np.random.default_rng(123)
    x = rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))
    # add exact midpoints between neighbours (ties) and values next to them
    i = rng.integers(1000, len(sv) - 1000, 4000)
    mids = (sv[i] + sv[i + 1]) / 2.0        # exact in fp64
    x = np.concatenate([x, mids, np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf)])
    got = f64_to_bf16(x)
    j = np.searchsorted(sv, x)  # sv[j-1] < x <= sv[j]
    lo, hi = sv[j - 1], sv[j]
    dlo, dhi = x - lo, hi - x                # exact: neighbours within a factor 2
    even_hi = (sb[j] & 1) == 0
    pick_hi = (dhi < dlo) | ((dhi == dlo) & even_hi)
    want = np.where(x == hi, sb[j], np.where(pick_hi, sb[j], sb[j - 1]))
    assert np.array_equal(got, want)


def test_rejects_out_of_contract():
    with pytest.raises(ValueError):
        f64_to_bf16(np.array([np.nan]))
    with pytest.raises(ValueError):
        f64_to_bf16(np.array([1e-40]))
