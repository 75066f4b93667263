"""Pins of the finer-scaling oracle (oracle/finer.py): a hand-worked golden case,
the scale invariance of per-row scaling, the largest element landing on the
format's maximum, degenerate rows, and a brute-force scaled GEMM in exact
rational arithmetic."""

import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import bf16 as obf16
from oracle import finer as ofin
from oracle import fp8 as ofp8
from oracle import gemm as ogemm

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "rowwise_current_e4m3.txt")


def _golden_rows():
    rows = []
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        x, a, s, c = (p.strip() for p in line.split("|"))
        rows.append((np.array([float(v) for v in x.split()], np.float32), float(a),
                     np.array([int(s, 16)], np.uint32).view(np.float32)[0],
                     np.array([int(v, 16) for v in c.split()], np.uint8)))
    return rows


def test_rowwise_golden_case():
    rows = _golden_rows()
    x = np.stack([r[0] for r in rows])
    codes, scale, sinv, amax = ofin.rowwise_cast(x, ofp8.E4M3, 0)
    for i, (_, a, s, c) in enumerate(rows):
        assert amax[i] == a and scale[i] == s
        np.testing.assert_array_equal(codes[i], c)
        assert sinv[i] == np.float32(np.float32(1) / s)


def test_margin_halves_the_scale():
    x = np.stack([r[0] for r in _golden_rows()])
    _, s0, _, _ = ofin.rowwise_cast(x, ofp8.E4M3, 0)
    codes1, s1, _, _ = ofin.rowwise_cast(x, ofp8.E4M3, 1)
    np.testing.assert_array_equal(s1, s0 / 2)
    assert codes1[0, 3] == 0x76  # 4 * 56 = 224


@pytest.mark.parametrize("fmt,top", [(ofp8.E4M3, 0x7E), (ofp8.E5M2, 0x7B)])
def test_power_of_two_rows_share_codes_and_max_lands_on_max(fmt, top):
    base = np.random.default_rng(3).standard_normal(64).astype(np.float32)
    base[17] = -3.0 * np.abs(base).max()  # the largest magnitude, negative
    x = np.stack([base * np.float32(2.0 ** e) for e in (-6, -1, 0, 3, 9)])
    codes, scale, _, amax = ofin.rowwise_cast(x, fmt, 0)
    for r in range(1, 5):
        np.testing.assert_array_equal(codes[r], codes[0])
    e = np.array([-6, -1, 0, 3, 9], dtype=np.float64)
    np.testing.assert_array_equal(scale.astype(np.float64) * 2.0 ** e, scale[2])
    assert (codes[:, 17] == (0x80 | top)).all()  # the row amax maps to -FP8_MAX
    assert (np.abs(ofp8.decode(codes, fmt)) <= ofp8.fmt_max(fmt)).all()


def test_per_row_not_per_tensor():
    x = np.array([[1.0, 0.5], [100.0, 50.0]], np.float32)
    codes, scale, _, _ = ofin.rowwise_cast(x, ofp8.E4M3, 0)
    np.testing.assert_array_equal(codes[0], codes[1])  # each row fills the range
    assert scale[0] == 448.0 and scale[1] == np.float32(4.48)


def test_degenerate_rows():
    x = np.zeros((3, 8), np.float32)
    x[1, 2] = np.inf
    x[2, 5] = np.nan
    codes, scale, sinv, amax = ofin.rowwise_cast(x, ofp8.E4M3, 0)
    np.testing.assert_array_equal(scale, [1.0, 1.0, 1.0])  # amax 0, inf, NaN -> 1.0
    np.testing.assert_array_equal(sinv, [1.0, 1.0, 1.0])
    assert not codes[0].any()
    assert codes[1, 2] == 0x7E and codes[2, 5] == 0x7F


def test_current_cast_is_one_row_of_rowwise():
    x = (np.random.default_rng(5).standard_normal((7, 33)) * 40).astype(np.float32)
    codes, s, a, sat = ofin.current_cast(x, ofp8.E5M2, 2)
    rc, rs, _, ra = ofin.rowwise_cast(x.reshape(1, -1), ofp8.E5M2, 2)
    np.testing.assert_array_equal(codes.ravel(), rc[0])
    assert s == rs[0] and a == ra[0] and sat == 0


def _exact_bf16(y: Fraction) -> np.uint16:
    """Round an exact rational to BF16 (nearest, ties to even) by its own
    arithmetic: the two BF16 neighbours of y are found from y's binade."""
    if y == 0:
        return np.uint16(0)
    sign = 0x8000 if y < 0 else 0
    a = abs(y)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp = Fraction(2) ** (e - 7)               # 8 significant bits
    lo = (a // ulp) * ulp
    rem = a - lo
    up = rem > ulp / 2 or (rem == ulp / 2 and (lo / ulp) % 2 == 1)
    v = float(lo + ulp if up else lo)
    bits = int(np.array([v], np.float32).view(np.uint32)[0] >> 16)
    return np.uint16(bits | sign)


def test_scaled_gemm_brute_force():
    """Exact rational evaluation of the pages' dequant (divide the product sum by
    the product of the two scales) at scales that are not powers of two."""
    rng = np.random.default_rng(9)
    M, K, N = 3, 5, 4
    a_codes = rng.integers(0, 256, (M, K), dtype=np.uint8)
    b_codes = rng.integers(0, 256, (N, K), dtype=np.uint8)  # stored [N, K], used as op T
    a_codes[(a_codes & 0x7F) == 0x7F] = 0x10                   # no NaN codes
    b_codes[(b_codes & 0x7F) >= 0x7C] = 0x22                   # no E5M2 inf / NaN codes
    sa = np.array([1.0, 4.48, 3.0], np.float32)
    sb = np.array([0.5, 57.344, 1.0 / 3.0, 7.0], np.float32)
    acc, _ = ogemm.gemm_exact(a_codes, ofp8.E4M3, ogemm.OP_N, b_codes, ofp8.E5M2, ogemm.OP_T)
    got = ofin.dequant_vec_to_bf16(acc, sa, sb)
    da = ofp8.decode(a_codes, ofp8.E4M3)
    db = ofp8.decode(b_codes, ofp8.E5M2)
    for i in range(M):
        for j in range(N):
            exact = sum(Fraction(float(da[i, k])) * Fraction(float(db[j, k])) for k in range(K))
            prod = Fraction(float(np.float32(sa[i] * sb[j])))  # one fp32 multiply
            assert got[i, j] == _exact_bf16(exact / prod), (i, j)


def test_dequant_is_a_division_not_reciprocal_products():
    """A pin that tells the pages' reading (divide by the scale product) from a
    kernel-style one (multiply by fl32(1/s_a) and fl32(1/s_b)).  Sums are placed
    2^-30 (relative) above or below a BF16 rounding midpoint of the quotient, at
    non-power-of-two scales: the oracle must equal the exact rational quotient
    rounded to BF16 on every case, while the reciprocal reading (relative error
    up to a few 2^-24) lands on the other side of the midpoint on some."""
    rng = np.random.default_rng(12)
    n = 400
    sa = (rng.uniform(1, 2, n) * 2.0 ** rng.integers(-6, 7, n)).astype(np.float32)
    sb = (rng.uniform(1, 2, n) * 3.0).astype(np.float32)
    hi = rng.integers(0x3F80, 0x4700, n).astype(np.uint32)       # BF16 values in [1, 2^15)
    lo_v = (hi << 16).view(np.float32).astype(np.float64)
    ulp = np.ldexp(1.0, np.frexp(lo_v)[1] - 8)                  # BF16 spacing at lo_v
    mid = lo_v + ulp / 2                                        # midpoint to the next value
    side = np.where(rng.integers(0, 2, n) == 1, 1.0, -1.0)
    prod = (sa * sb).astype(np.float32).astype(np.float64)
    acc = mid * (1.0 + side * 2.0**-30) * prod
    got = np.array([ofin.dequant_vec_to_bf16(acc[i:i + 1, None], sa[i:i + 1], sb[i:i + 1])[0, 0]
                    for i in range(n)], np.uint16)
    exact = np.array([_exact_bf16(Fraction(float(acc[i])) / Fraction(float(prod[i])))
                      for i in range(n)], np.uint16)
    np.testing.assert_array_equal(got, exact)
    recip = obf16.round_to_bf16_vec(
        acc * np.array([np.float64(ofin.inv_scale(s)) for s in sa]) *
        np.array([np.float64(ofin.inv_scale(s)) for s in sb]))
    assert (recip != exact).sum() >= n // 20


def test_scaled_gemm_reduces_to_per_tensor_for_equal_scales():
    """Equal scales along rows and columns give the per-tensor dequant exactly."""
    rng = np.random.default_rng(11)
    a_codes = rng.integers(0, 0x7E, (8, 16), dtype=np.uint8)
    b_codes = rng.integers(0, 0x7E, (16, 6), dtype=np.uint8)
    acc, _ = ogemm.gemm_exact(a_codes, ofp8.E4M3, ogemm.OP_N, b_codes, ofp8.E4M3, ogemm.OP_N)
    for sa, sb in ((np.float32(64.0), np.float32(0.5)), (np.float32(4.48), np.float32(57.344))):
        per_tensor = ogemm.dequant_to_bf16(acc, sa, sb)
        vec = ofin.dequant_vec_to_bf16(acc, np.full(8, sa, np.float32), np.full(6, sb, np.float32))
        np.testing.assert_array_equal(per_tensor, vec)
