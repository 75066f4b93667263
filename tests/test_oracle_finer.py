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


def test_scaled_gemm_brute_force():
    rng = np.random.default_rng(9)
    M, K, N = 3, 5, 4
    a_codes = rng.integers(0, 256, (M, K), dtype=np.uint8)
    b_codes = rng.integers(0, 256, (N, K), dtype=np.uint8)  # stored [N, K], used as op T
    a_codes[(a_codes & 0x7F) == 0x7F] = 0x10                   # no NaN codes
    b_codes[(b_codes & 0x7F) >= 0x7C] = 0x22                   # no E5M2 inf / NaN codes
    ia = np.array([1.0, 0.25, 3.0], np.float32)
    ib = np.array([0.5, 2.0, 1.0 / 3.0, 7.0], np.float32)
    acc, _ = ogemm.gemm_exact(a_codes, ofp8.E4M3, ogemm.OP_N, b_codes, ofp8.E5M2, ogemm.OP_T)
    got = ofin.dequant_vec_to_bf16(acc, ia, ib)
    da = ofp8.decode(a_codes, ofp8.E4M3)
    db = ofp8.decode(b_codes, ofp8.E5M2)
    for i in range(M):
        for j in range(N):
            exact = sum(Fraction(float(da[i, k])) * Fraction(float(db[j, k])) for k in range(K))
            y = exact * Fraction(float(ia[i])) * Fraction(float(ib[j]))
            assert got[i, j] == obf16.round_to_bf16_vec(np.array([float(y)]))[0], (i, j)


def test_scaled_gemm_reduces_to_per_tensor_for_power_of_two_scales():
    rng = np.random.default_rng(11)
    a_codes = rng.integers(0, 0x7E, (8, 16), dtype=np.uint8)
    b_codes = rng.integers(0, 0x7E, (16, 6), dtype=np.uint8)
    acc, _ = ogemm.gemm_exact(a_codes, ofp8.E4M3, ogemm.OP_N, b_codes, ofp8.E4M3, ogemm.OP_N)
    sa, sb = np.float32(64.0), np.float32(0.5)
    per_tensor = ogemm.dequant_to_bf16(acc, sa, sb)
    vec = ofin.dequant_vec_to_bf16(acc, np.full(8, 1 / sa, np.float32), np.full(6, 1 / sb, np.float32))
    np.testing.assert_array_equal(per_tensor, vec)
